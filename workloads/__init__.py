"""Seeded synthetic inputs for sparse MLA prefill attention.

Shared by the tests, the smoke check and the benchmark.  This module only
draws inputs; it holds none of the attention's arithmetic (no dequantisation,
no dot products, no softmax).  Shapes follow the DeepSeek-V3.2 MLA workload
described on the "mla_sm100_prefill_sparse_fp8" page (128 query heads, qk
depth 576 = 512 + 64 rope, v depth 512, FP8 e4m3fn latent cache, BF16 q/out,
uint32 indices with a per-query effective top-k count).

Draw order for one case, all from one torch.Generator seeded with `seed` on
the target device: q, scales, latent, page permutation, topk lengths,
indices, sink.  Indices of a query at sequence position `pos` are distinct
and drawn uniformly from its causal prefix [0, pos] in random order; slots at
or beyond the effective count hold 0xFFFFFFFF.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

QK_DEPTH = 576
V_DEPTH = 512
PAD_INDEX = 0xFFFFFFFF


@dataclasses.dataclass(frozen=True)
class CaseSpec:
    name: str
    num_seqs: int            # B
    q_per_seq: int           # query tokens per sequence
    ctx: int                 # KV context length per sequence (tokens)
    q_pos0: int              # position of the first query token of each sequence
    num_heads: int
    topk: int                # indices row stride (K)
    page_size: int = 64
    scale_block_size: int = 0        # 0 unit, >= 576 tensorwise, else blockwise
    sink: bool = False
    shuffle_pages: bool = False      # random physical page permutation
    lengths: str = "causal"          # "causal": min(K, pos+1); "uniform:lo:hi"; "full": K
    spare_pages: int = 0             # extra physical pages no table references
    poison: bool = False             # fill spare pages with the NaN byte 0x7F
    scale_lo_log2: float = -4.0      # per-row / per-block scales are 2^U(lo, hi)
    scale_hi_log2: float = 2.0
    softmax_scale: float = 192.0 ** -0.5

    @property
    def num_tokens(self) -> int:
        return self.num_seqs * self.q_per_seq

    @property
    def pages_per_seq(self) -> int:
        return -(-self.ctx // self.page_size)

    @property
    def num_pages(self) -> int:
        return self.num_seqs * self.pages_per_seq + self.spare_pages

    @property
    def scale_cols(self) -> int:
        if self.scale_block_size == 0:
            return 0
        if self.scale_block_size >= QK_DEPTH:
            return 1
        return -(-QK_DEPTH // self.scale_block_size)


# The five workloads: a tiny one the oracle finishes in seconds, the DSv3.2
# prefill shape, tensorwise scales with a sink, blockwise scales with ragged
# lengths and permuted pages, and the decode/MTP shape.  Where a workload does
# not fix the query positions, queries sit at the end of their context.
CONFIGS = {
    "tiny": CaseSpec("tiny", num_seqs=1, q_per_seq=16, ctx=256, q_pos0=240, num_heads=16,
                     topk=64, lengths="full"),
    "dsv32": CaseSpec("dsv32", num_seqs=1, q_per_seq=4096, ctx=8192, q_pos0=4096, num_heads=128,
                      topk=2048),
    "tensor_sink": CaseSpec("tensor_sink", num_seqs=4, q_per_seq=2048, ctx=4096, q_pos0=2048,
                            num_heads=64, topk=2048, scale_block_size=576, sink=True),
    "blockwise": CaseSpec("blockwise", num_seqs=2, q_per_seq=8192, ctx=16384, q_pos0=8192,
                          num_heads=128, topk=2048, scale_block_size=32, shuffle_pages=True,
                          lengths="uniform:512:2048"),
    "decode": CaseSpec("decode", num_seqs=64, q_per_seq=2, ctx=32768, q_pos0=32766,
                       num_heads=128, topk=2048, shuffle_pages=True),
}

SEEDS = {"tiny": 1001, "dsv32": 1002, "tensor_sink": 1003, "blockwise": 1004, "decode": 1005}


@dataclasses.dataclass
class Case:
    spec: CaseSpec
    q: torch.Tensor                 # bf16 [T, H, 576]
    kv_pages: torch.Tensor          # uint8 [num_pages, P, 576] (e4m3fn codes)
    page_table: torch.Tensor        # int32 [B, pages_per_seq]
    cu_seqlens_q: torch.Tensor      # int32 [B + 1]
    scales: Optional[torch.Tensor]  # float32 [num_pages * P, ncols] or None
    indices: torch.Tensor           # int32 [T, K] holding uint32 bit patterns
    topk_lengths: torch.Tensor      # int32 [T] (uint32 values)
    sink: Optional[torch.Tensor]    # float32 [H] or None
    positions: torch.Tensor         # int64 [T] position of each query in its sequence
    scale: float
    scale_block_size: int

    def to(self, device) -> "Case":
        def mv(x):
            return None if x is None else x.to(device)
        return dataclasses.replace(
            self, q=mv(self.q), kv_pages=mv(self.kv_pages), page_table=mv(self.page_table),
            cu_seqlens_q=mv(self.cu_seqlens_q), scales=mv(self.scales), indices=mv(self.indices),
            topk_lengths=mv(self.topk_lengths), sink=mv(self.sink), positions=mv(self.positions))

    def host_arrays(self) -> dict:
        """numpy views for the oracle (uint16 q patterns, uint8 codes, ...)."""
        import numpy as np
        return {
            "q_bits": self.q.cpu().view(torch.int16).numpy().view(np.uint16),
            "kv_pages": self.kv_pages.cpu().numpy(),
            "page_table": self.page_table.cpu().numpy(),
            "cu_seqlens_q": self.cu_seqlens_q.cpu().numpy(),
            "scales": None if self.scales is None else self.scales.cpu().numpy(),
            "indices": self.indices.cpu().numpy().view(np.uint32),
            "topk_lengths": self.topk_lengths.cpu().numpy().view(np.uint32),
            "sink": None if self.sink is None else self.sink.cpu().numpy(),
            "scale": self.scale,
            "scale_block_size": self.scale_block_size,
        }


def _fp8_codes(x: torch.Tensor) -> torch.Tensor:
    """Round to e4m3fn (saturating at +-448 first) and return the byte codes."""
    return x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def make_case(spec: CaseSpec, seed: int, device="cpu", chunk_rows: int = 1 << 20) -> Case:
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    T, H, B, P, K = spec.num_tokens, spec.num_heads, spec.num_seqs, spec.page_size, spec.topk
    num_rows = spec.num_pages * P

    # q ~ N(0, 1) rounded to bf16
    q = torch.empty((T, H, QK_DEPTH), dtype=torch.bfloat16, device=device)
    step = max(1, (1 << 24) // (H * QK_DEPTH))
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        q[t0:t1] = torch.randn((t1 - t0, H, QK_DEPTH), generator=g, device=device).to(torch.bfloat16)

    # scales 2^U(lo, hi), one per row or one per (row, block)
    ncols = spec.scale_cols
    scales = None
    if ncols:
        u = torch.rand((num_rows, ncols), generator=g, device=device, dtype=torch.float64)
        scales = torch.exp2(spec.scale_lo_log2 + (spec.scale_hi_log2 - spec.scale_lo_log2) * u).to(torch.float32)

    # latent = e4m3fn(x / scale), x ~ N(0, 1)
    kv = torch.empty((num_rows, QK_DEPTH), dtype=torch.uint8, device=device)
    if ncols:
        col_block = torch.arange(QK_DEPTH, device=device) // spec.scale_block_size if ncols > 1 else None
    for r0 in range(0, num_rows, chunk_rows):
        r1 = min(num_rows, r0 + chunk_rows)
        x = torch.randn((r1 - r0, QK_DEPTH), generator=g, device=device)
        if ncols == 1:
            x = x / scales[r0:r1, 0:1]
        elif ncols > 1:
            x = x / scales[r0:r1][:, col_block]
        kv[r0:r1] = _fp8_codes(x)

    # page table: sequence b owns pages_per_seq physical pages
    pps = spec.pages_per_seq
    if spec.shuffle_pages:
        perm = torch.randperm(spec.num_pages, generator=g, device=device)
    else:
        perm = torch.arange(spec.num_pages, device=device)
    used = perm[: B * pps]
    spare = perm[B * pps:]
    page_table = used.reshape(B, pps).to(torch.int32)
    kv = kv.reshape(spec.num_pages, P, QK_DEPTH)
    if spec.poison and spare.numel():
        kv[spare] = 0x7F

    cu = torch.arange(0, (B + 1) * spec.q_per_seq, spec.q_per_seq, dtype=torch.int32, device=device)
    positions = (spec.q_pos0 + torch.arange(spec.q_per_seq, device=device)).repeat(B).to(torch.int64)

    # effective top-k counts
    prefix = positions + 1
    if spec.lengths == "causal":
        lengths = torch.clamp(prefix, max=K)
    elif spec.lengths == "full":
        lengths = torch.full((T,), K, dtype=torch.int64, device=device)
    elif spec.lengths.startswith("uniform:"):
        _, lo, hi = spec.lengths.split(":")
        lengths = torch.randint(int(lo), int(hi) + 1, (T,), generator=g, device=device)
        lengths = torch.minimum(lengths, prefix)
    else:
        raise ValueError(spec.lengths)

    # indices: distinct, uniform over the causal prefix, random order
    indices = torch.full((T, K), -1, dtype=torch.int32, device=device)   # 0xFFFFFFFF
    ctx = spec.ctx
    tstep = max(1, (1 << 24) // ctx)
    col = torch.arange(ctx, device=device)
    kk = torch.arange(K, device=device)
    for t0 in range(0, T, tstep):
        t1 = min(T, t0 + tstep)
        r = torch.rand((t1 - t0, ctx), generator=g, device=device)
        r = torch.where(col[None, :] <= positions[t0:t1, None], r, torch.full_like(r, 2.0))
        kq = min(K, ctx)
        sel = torch.topk(r, kq, dim=1, largest=False).indices.to(torch.int32)
        blk = torch.full((t1 - t0, K), -1, dtype=torch.int32, device=device)
        blk[:, :kq] = sel
        keep = kk[None, :] < lengths[t0:t1, None]
        indices[t0:t1] = torch.where(keep, blk, torch.full_like(blk, -1))

    sink = None
    if spec.sink:
        sink = torch.randn((H,), generator=g, device=device).to(torch.float32)

    return Case(spec=spec, q=q, kv_pages=kv, page_table=page_table, cu_seqlens_q=cu,
                scales=scales, indices=indices, topk_lengths=lengths.to(torch.int32), sink=sink,
                positions=positions, scale=spec.softmax_scale,
                scale_block_size=spec.scale_block_size)


def subset_host_arrays(case: Case, tokens, cache: dict = None) -> dict:
    """Host (numpy) inputs for a subset of tokens, each re-expressed as a
    one-token sequence over its own page-table row (pure slicing).  `cache`
    (a dict kept by the caller) holds the host copies of the token-independent
    arrays across calls."""
    import numpy as np
    tokens = np.asarray(tokens, dtype=np.int64)
    tix = torch.from_numpy(tokens).to(case.q.device)
    if cache is None:
        cache = {}
    if "kv_pages" not in cache:
        cache["kv_pages"] = case.kv_pages.cpu().numpy()
        cache["page_table"] = case.page_table.cpu().numpy()
        cache["cu"] = case.cu_seqlens_q.cpu().numpy()
        cache["scales"] = None if case.scales is None else case.scales.cpu().numpy()
    seq_of = np.searchsorted(cache["cu"], tokens, side="right") - 1
    return {
        "q_bits": case.q[tix].cpu().view(torch.int16).numpy().view(np.uint16),
        "kv_pages": cache["kv_pages"],
        "page_table": cache["page_table"][seq_of],
        "cu_seqlens_q": np.arange(len(tokens) + 1, dtype=np.int32),
        "scales": cache["scales"],
        "indices": case.indices[tix].cpu().numpy().view(np.uint32),
        "topk_lengths": case.topk_lengths[tix].cpu().numpy().view(np.uint32),
        "sink": None if case.sink is None else case.sink.cpu().numpy(),
        "scale": case.scale,
        "scale_block_size": case.scale_block_size,
    }


def flops_of(case: Case, tokens=None) -> float:
    """Counted work: 2 * H * (576 + 512) FLOP per gathered key."""
    lens = case.topk_lengths.to(torch.int64)
    if tokens is not None:
        lens = lens[torch.as_tensor(tokens, device=lens.device)]
    L = torch.clamp(lens, max=case.spec.topk).sum().item()
    return 2.0 * case.spec.num_heads * (QK_DEPTH + V_DEPTH) * L


def scaled(spec: CaseSpec, **kw) -> CaseSpec:
    return dataclasses.replace(spec, **kw)


# --------------------------------------------------------------------------
# FP8 lightning indexer inputs (page "sparse_index_fp8_sm100": q [tokens,
# heads, 128] and paged keys [keys, 128] in FP8 e4m3 with a per-(token, head)
# q_scale and a per-key k_scale)
# --------------------------------------------------------------------------

INDEX_DEPTH = 128


@dataclasses.dataclass(frozen=True)
class IndexerSpec:
    name: str
    num_seqs: int
    q_per_seq: int
    ctx: int                      # keys per sequence (seq_lens_k)
    num_heads: int = 64
    topk: int = 2048
    page_size: int = 64
    shuffle_pages: bool = False
    spare_pages: int = 0
    score_stride: int = 0         # 0: ctx

    @property
    def num_tokens(self) -> int:
        return self.num_seqs * self.q_per_seq

    @property
    def pages_per_seq(self) -> int:
        return -(-self.ctx // self.page_size)

    @property
    def num_pages(self) -> int:
        return self.num_seqs * self.pages_per_seq + self.spare_pages

    @property
    def stride(self) -> int:
        return self.score_stride or self.ctx


INDEXER_CONFIGS = {
    "indexer_tiny": IndexerSpec("indexer_tiny", num_seqs=1, q_per_seq=16, ctx=256, topk=64),
    # the DSv3.2 prefill above: 4096 queries at positions 4096..8191 of one sequence
    "indexer_dsv32": IndexerSpec("indexer_dsv32", num_seqs=1, q_per_seq=4096, ctx=8192, topk=2048),
}

INDEXER_SEEDS = {"indexer_tiny": 2001, "indexer_dsv32": 2002}


@dataclasses.dataclass
class IndexerCase:
    spec: IndexerSpec
    q: torch.Tensor             # uint8 [T, H, 128] e4m3fn codes
    q_scale: torch.Tensor       # float32 [T, H]
    k_pages: torch.Tensor       # uint8 [num_pages, P, 128] e4m3fn codes
    k_scale: torch.Tensor       # float32 [num_pages * P]
    page_table: torch.Tensor    # int32 [B, pages_per_seq]
    cu_seqlens_q: torch.Tensor  # int32 [B + 1]
    seq_lens_k: torch.Tensor    # int32 [B]

    def to(self, device) -> "IndexerCase":
        f = {k.name: getattr(self, k.name) for k in dataclasses.fields(self)}
        for k, v in f.items():
            if isinstance(v, torch.Tensor):
                f[k] = v.to(device)
        return IndexerCase(**f)

    def host_arrays(self) -> dict:
        import numpy as np
        return {
            "q_codes": self.q.cpu().numpy(), "q_scale": self.q_scale.cpu().numpy(),
            "k_pages": self.k_pages.cpu().numpy(), "k_scale": self.k_scale.cpu().numpy(),
            "page_table": self.page_table.cpu().numpy(), "cu_seqlens_q": self.cu_seqlens_q.cpu().numpy(),
            "seq_lens_k": self.seq_lens_k.cpu().numpy(),
        }


def make_indexer_case(spec: IndexerSpec, seed: int, device="cpu", q_lens=None) -> IndexerCase:
    """Draw order: q, q_scale, keys, page permutation.  Keys are quantised per
    row (k_scale = max|row| / 448, codes = e4m3(row / k_scale)), q codes are
    e4m3 of N(0, 1) x 32, q_scale ~ N(0, 1) / (32 sqrt(H)).  `q_lens`
    (optional, per sequence) overrides q_per_seq for ragged batches."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    B, H, P = spec.num_seqs, spec.num_heads, spec.page_size
    lens = [spec.q_per_seq] * B if q_lens is None else list(q_lens)
    T = sum(lens)
    q = _fp8_codes(torch.randn((T, H, INDEX_DEPTH), generator=g, device=device) * 32.0)
    q_scale = (torch.randn((T, H), generator=g, device=device) / (32.0 * math.sqrt(H))).to(torch.float32)
    rows = spec.num_pages * P
    x = torch.randn((rows, INDEX_DEPTH), generator=g, device=device)
    k_scale = (x.abs().amax(dim=1) / 448.0).clamp_min(1e-8).to(torch.float32)
    k = _fp8_codes(x / k_scale[:, None]).reshape(spec.num_pages, P, INDEX_DEPTH)
    if spec.shuffle_pages:
        perm = torch.randperm(spec.num_pages, generator=g, device=device)
    else:
        perm = torch.arange(spec.num_pages, device=device)
    page_table = perm[: B * spec.pages_per_seq].reshape(B, spec.pages_per_seq).to(torch.int32)
    cu = torch.zeros(B + 1, dtype=torch.int32, device=device)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int32, device=device), 0)
    seq_lens_k = torch.full((B,), spec.ctx, dtype=torch.int32, device=device)
    return IndexerCase(spec=spec, q=q, q_scale=q_scale, k_pages=k, k_scale=k_scale, page_table=page_table,
                       cu_seqlens_q=cu, seq_lens_k=seq_lens_k)


def indexer_flops(case: IndexerCase) -> float:
    """Counted work: 2 * H * 128 FLOP per (query token, visible key)."""
    cu = case.cu_seqlens_q.cpu().tolist()
    lk = case.seq_lens_k.cpu().tolist()
    stride = case.spec.stride
    total = 0
    for b in range(len(lk)):
        q_len = cu[b + 1] - cu[b]
        for i in range(q_len):
            total += min(max(lk[b] - q_len + i + 1, 0), stride)
    return 2.0 * case.spec.num_heads * INDEX_DEPTH * total


# ---------------------------------------------------------------- dense MLA prefill

@dataclasses.dataclass(frozen=True)
class DenseSpec:
    name: str
    num_seqs: int
    max_prompt_len: int           # S: rows per sequence in q and out
    lengths: tuple = ()           # valid_length per sequence (default: all S)
    num_heads: int = 128
    num_kv_heads: int = 0         # 0: num_heads
    page_size: int = 64
    scale_block_size: int = 32    # K_rope scales: 0 unit, >= 64 per row, 16 / 32 / 48 per block
    causal: bool = True
    shuffle_pages: bool = True
    spare_pages: int = 0

    @property
    def kv_heads(self) -> int:
        return self.num_kv_heads or self.num_heads

    @property
    def pages_per_seq(self) -> int:
        return -(-self.max_prompt_len // self.page_size)

    @property
    def num_pages(self) -> int:
        return self.num_seqs * self.pages_per_seq + self.spare_pages

    @property
    def valid_lengths(self) -> tuple:
        return tuple(self.lengths) if self.lengths else (self.max_prompt_len,) * self.num_seqs

    @property
    def scale_cols(self) -> int:
        s = self.scale_block_size
        return 0 if s == 0 else (1 if s >= 64 else -(-64 // s))


# A small case the oracle finishes in seconds, and the DeepSeek-V3 prefill
# shape: 128 heads, q 192 = 128 nope + 64 rope, v 128, two 4096-token prompts.
DENSE_CONFIGS = {
    "dense_tiny": DenseSpec("dense_tiny", num_seqs=2, max_prompt_len=200, lengths=(200, 131), num_heads=4,
                            page_size=16),
    "dense_dsv3": DenseSpec("dense_dsv3", num_seqs=2, max_prompt_len=4096, num_heads=128),
}
DENSE_SEEDS = {"dense_tiny": 3001, "dense_dsv3": 3002}


@dataclasses.dataclass
class DenseCase:
    spec: DenseSpec
    q: torch.Tensor               # bf16 [B * S, H, 192]
    k_nope: torch.Tensor          # bf16 [num_pages, P, Hkv, 128]
    v: torch.Tensor               # bf16 [num_pages, P, Hkv, 128]
    k_rope: torch.Tensor          # uint8 [num_pages, P, 64] e4m3fn codes
    k_rope_scales: Optional[torch.Tensor]   # float32 [num_pages * P, ncols]
    page_table: torch.Tensor      # int32 [B, pages_per_seq]
    valid_length: torch.Tensor    # int32 [B]
    scale: float

    def to(self, device) -> "DenseCase":
        f = {k.name: getattr(self, k.name) for k in dataclasses.fields(self)}
        for k, v in f.items():
            if isinstance(v, torch.Tensor):
                f[k] = v.to(device)
        return DenseCase(**f)

    def host_arrays(self) -> dict:
        import numpy as np
        s = self.spec
        return {
            "q_bits": self.q.cpu().view(torch.int16).numpy().view(np.uint16),
            "k_nope_bits": self.k_nope.cpu().view(torch.int16).numpy().view(np.uint16),
            "v_bits": self.v.cpu().view(torch.int16).numpy().view(np.uint16),
            "k_rope_codes": self.k_rope.cpu().numpy(),
            "k_rope_scales": None if self.k_rope_scales is None else self.k_rope_scales.cpu().numpy(),
            "page_table": self.page_table.cpu().numpy(),
            "valid_length": self.valid_length.cpu().numpy().view(np.uint32),
            "scale": self.scale, "scale_block_size": s.scale_block_size, "max_prompt_len": s.max_prompt_len,
            "causal": s.causal,
        }


def make_dense_case(spec: DenseSpec, seed: int, device="cpu") -> DenseCase:
    """Draw order: q, K_nope, V, K_rope, page permutation.  q, K_nope and V are
    bf16 of N(0, 1); K_rope rows are x ~ N(0, 1) quantised with block scales
    2^U(-4, 2): codes = e4m3(x / scale) (scales 1 with scale_block_size 0).
    Softmax scale 192^-0.5."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    B, S, H, Hkv, P = spec.num_seqs, spec.max_prompt_len, spec.num_heads, spec.kv_heads, spec.page_size
    NP = spec.num_pages
    q = torch.randn((B * S, H, 192), generator=g, device=device).to(torch.bfloat16)
    k_nope = torch.randn((NP, P, Hkv, 128), generator=g, device=device).to(torch.bfloat16)
    v = torch.randn((NP, P, Hkv, 128), generator=g, device=device).to(torch.bfloat16)
    x = torch.randn((NP * P, 64), generator=g, device=device)
    nc = spec.scale_cols
    if nc == 0:
        scales = None
        k_rope = _fp8_codes(x)
    else:
        # log-uniform, not powers of two, so fp8 * scale really rounds to bf16
        u = torch.rand((NP * P, nc), generator=g, device=device, dtype=torch.float64)
        scales = torch.exp2(-4.0 + 6.0 * u).to(torch.float32)
        blk = 64 if spec.scale_block_size >= 64 else spec.scale_block_size
        col = torch.arange(64, device=device) // blk
        k_rope = _fp8_codes(x / scales[:, col])
    k_rope = k_rope.reshape(NP, P, 64)
    if spec.shuffle_pages:
        perm = torch.randperm(NP, generator=g, device=device)
    else:
        perm = torch.arange(NP, device=device)
    page_table = perm[: B * spec.pages_per_seq].reshape(B, spec.pages_per_seq).to(torch.int32)
    valid_length = torch.tensor(spec.valid_lengths, dtype=torch.int32, device=device)
    return DenseCase(spec=spec, q=q, k_nope=k_nope, v=v, k_rope=k_rope, k_rope_scales=scales,
                     page_table=page_table, valid_length=valid_length, scale=192 ** -0.5)


def dense_flops(spec: DenseSpec) -> float:
    """Counted work: 2 * H * (192 + 128) FLOP per visible (row, key) pair."""
    pairs = 0
    for L in spec.valid_lengths:
        L = min(int(L), spec.max_prompt_len)
        pairs += L * (L + 1) // 2 if spec.causal else L * L
    return 2.0 * spec.num_heads * (192 + 128) * pairs
