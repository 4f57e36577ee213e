"""CPU float64 oracle for sparse MLA prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, table or helper with the HIP
library: it has its own FP8/bf16 decoders and its own page translation.

What it computes (the plain definition, written out, no blocking or fusion):

  For query token t of sequence b and head h, with L = min(topk_lengths[t], K):
    row_j  = page_table[b, idx_j // P] * P + idx_j % P   for slots j < L
    k_j[c] = dec_e4m3fn(kv[row_j, c]) * sigma(row_j, c)   c in [0, 576)
    v_j    = k_j[0:512]
    s_j    = scale * sum_c q[t,h,c] * k_j[c]
    Z      = sum_j exp(s_j) (+ exp(sink_h) when a sink is given)
    out    = sum_j exp(s_j) / Z * v_j

Sources (Modular kernel API docs):
  * "mla_sm100_prefill_sparse_fp8" page -- Args: output [total_q_tokens,
    num_q_heads, v_depth], q [total_q_tokens, num_q_heads, qk_depth], paged
    float8_e4m3fn kv_cache, per-query uint32 indices with topk_lengths as the
    effective top-k count, optional attention sink, scales_ptr laid out
    [total_phys_rows, ceildiv(qk_depth, scale_block_size)] in physical-row
    space, softmax scale.  Parameters: num_q_heads 128, qk_depth 576,
    v_depth 512, indices_stride = top-k count, and the three scale modes of
    scale_block_size (0: unit scale, >= qk_depth: one scale per KV row,
    smaller: blockwise, K using all ceildiv(qk_depth, sbs) blocks and V the
    first ceildiv(v_depth, sbs)).
  * "mla_prefill_sparse_qkv_fp8" page -- K and V share the MLA latent; V is
    the first v_depth columns of the same gathered rows.
  * "SM100MLA" page -- cache_depth 576 with a 64-column rope part, f32
    accumulation, softmax with a running max ("correction") and a final
    1/row_sum scaling of the output.
  * "mla_sm100_prefill_blockscale" page -- the softmax scale multiplies the
    Q.K' dot product.

Readings where the pages are silent (each is listed with its reason in the
project's design notes):
  * indices are logical positions inside the token's own sequence and pass
    through page_table; scales are indexed by physical row;
  * the sink is a per-head logit in the same natural-log units as s_j; it adds
    exp(sink_h) to the denominator only and carries no value;
  * slots j >= L are never read; a slot whose index or page id is out of range
    is masked (weight 0); L is clamped to K; an empty key set gives out = 0;
  * duplicate indices count with multiplicity; no causal mask is applied here
    (the index list is the key set).
"""

from __future__ import annotations

import numpy as np

QK_DEPTH = 576   # "SM100MLA" page: cache_depth
V_DEPTH = 512    # "mla_sm100_prefill_sparse_fp8" page: v_depth for DSv3.2


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """Decode OCP float8 e4m3fn byte codes to float64.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
    field 0 is subnormal (m/8 * 2^-6).  There is no infinity; S.1111.111 is
    NaN.  The kv_cache dtype is DType.float8_e4m3fn on the
    "mla_prefill_sparse_qkv_fp8" page (FP8_TYPE) and the
    "mla_sm100_prefill_sparse_fp8" page (cache_t).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64.

    bfloat16 is the top half of an IEEE binary32, so widening the pattern by
    16 zero bits gives the exact binary32 value.  q and output are BF16 on the
    "mla_sm100_prefill_sparse_fp8" page (q_type, output_type).
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Index translation (paged cache)
# --------------------------------------------------------------------------

def token_sequences(cu_seqlens_q: np.ndarray, num_tokens: int) -> np.ndarray:
    """Sequence id of every packed query token, from the [B+1] offsets."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    seq = np.full(num_tokens, -1, dtype=np.int64)
    for b in range(len(cu) - 1):
        seq[cu[b]:cu[b + 1]] = b
    return seq


def translate_rows(indices, topk_lengths, page_table, cu_seqlens_q,
                   page_size: int, num_pages: int, tokens=None) -> np.ndarray:
    """Physical KV row of every listed slot, -1 where the slot is not read.

    Follows the "mla_sm100_prefill_sparse_fp8" page: indices are per-query
    uint32 slots, topk_lengths the effective count per query, and the cache is
    paged (scales in physical-row space).  Reading: idx is a logical position
    in the token's sequence; row = page_table[b, idx // P] * P + idx % P.
    A slot is read only if j < min(topk_lengths[t], K), idx // P is inside
    the page-table row and the page id is in [0, num_pages).
    """
    indices = np.asarray(indices).astype(np.uint32).astype(np.int64)
    lengths = np.asarray(topk_lengths).astype(np.uint32).astype(np.int64)
    page_table = np.asarray(page_table, dtype=np.int64)
    T, K = indices.shape
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    seq = token_sequences(cu_seqlens_q, T)
    max_pages = page_table.shape[1]
    rows = np.full((len(tokens), K), -1, dtype=np.int64)
    for out_i, t in enumerate(tokens):
        b = seq[t]
        L = min(int(lengths[t]), K)
        if b < 0 or L <= 0:
            continue
        idx = indices[t, :L]
        logical_page = idx // page_size
        in_table = logical_page < max_pages
        pg = np.full(L, -1, dtype=np.int64)
        pg[in_table] = page_table[b, logical_page[in_table]]
        ok = in_table & (pg >= 0) & (pg < num_pages)
        r = pg * page_size + idx % page_size
        rows[out_i, :L] = np.where(ok, r, -1)
    return rows


def gather_rows(kv_pages: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Raw latent bytes of the listed rows ([n, K, 576] uint8), zero where
    the slot is not read.  kv_pages is [num_pages, P, 576] uint8."""
    flat = np.asarray(kv_pages, dtype=np.uint8).reshape(-1, kv_pages.shape[-1])
    out = np.zeros(rows.shape + (flat.shape[1],), dtype=np.uint8)
    ok = rows >= 0
    out[ok] = flat[rows[ok]]
    return out


# --------------------------------------------------------------------------
# Dequantisation (three scale modes)
# --------------------------------------------------------------------------

def dequant_rows(codes: np.ndarray, rows: np.ndarray, scales, scale_block_size: int) -> np.ndarray:
    """Dequantise raw latent rows to float64.

    "mla_sm100_prefill_sparse_fp8" page, Parameters: scale_block_size.
      0                      -> unit scale, scales unused;
      >= qk_depth            -> one scale per physical KV row;
      0 < sbs < qk_depth     -> block c // sbs of scales[row, :], the table
                                having ceildiv(qk_depth, sbs) columns.
    codes: [n, D] uint8, rows: [n] physical row ids (>= 0).
    """
    x = decode_e4m3fn(codes)
    D = codes.shape[-1]
    if scale_block_size == 0:
        return x
    s = np.asarray(scales, dtype=np.float64)
    if scale_block_size >= D:
        return x * s[rows, 0][:, None]
    block_of_col = np.arange(D) // scale_block_size
    return x * s[rows][:, block_of_col]


# --------------------------------------------------------------------------
# The attention
# --------------------------------------------------------------------------

def sparse_mla_prefill(q_bits, kv_pages, page_table, cu_seqlens_q, scales, indices,
                       topk_lengths, sink, scale: float, scale_block_size: int,
                       tokens=None, v_depth: int = V_DEPTH):
    """Sparse MLA prefill attention in float64 for the selected tokens.

    Arguments mirror the C-ABI entry point (host arrays):
      q_bits       uint16 [T, H, 576]  bf16 patterns
      kv_pages     uint8  [num_pages, P, 576]  e4m3fn codes
      page_table   int32  [B, max_pages_per_seq]
      cu_seqlens_q int32  [B + 1]
      scales       float32 [num_pages * P, ncols] or None (sbs == 0)
      indices      uint32 [T, K];  topk_lengths uint32 [T]
      sink         float32 [H] or None
    Returns a dict with, for the selected tokens:
      out          [n, H, v_depth] float64
      weight_sum   [n, H]  sum of the key weights exp(s_j)/Z
      sink_weight  [n, H]  exp(sink_h)/Z (0 without a sink)
      lse          [n, H]  log Z (-inf for an empty set without a sink)
      rows         [n, K]  physical rows read (-1 = not read)
    """
    q_bits = np.asarray(q_bits)
    T, H, D = q_bits.shape
    kv_pages = np.asarray(kv_pages, dtype=np.uint8)
    num_pages, P, _ = kv_pages.shape
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    rows = translate_rows(indices, topk_lengths, page_table, cu_seqlens_q, P, num_pages, tokens)
    flat = kv_pages.reshape(-1, D)
    sink64 = None if sink is None else np.asarray(sink, dtype=np.float64)

    n = len(tokens)
    out = np.zeros((n, H, v_depth))
    wsum = np.zeros((n, H))
    swgt = np.zeros((n, H))
    lse = np.full((n, H), -np.inf)
    for i, t in enumerate(tokens):
        valid = rows[i][rows[i] >= 0]
        q = decode_bf16(q_bits[t])                      # [H, 576]
        if valid.size == 0:
            if sink64 is not None:
                swgt[i] = 1.0
                lse[i] = sink64
            continue
        k = dequant_rows(flat[valid], valid, scales, scale_block_size)   # [n_valid, 576]
        v = k[:, :v_depth]
        s = scale * (q @ k.T)                            # [H, n_valid]
        m = s.max(axis=1)
        if sink64 is not None:
            m = np.maximum(m, sink64)
        w = np.exp(s - m[:, None])
        Z = w.sum(axis=1)
        if sink64 is not None:
            ws = np.exp(sink64 - m)
            Z = Z + ws
            swgt[i] = ws / Z
        p = w / Z[:, None]
        out[i] = p @ v
        wsum[i] = p.sum(axis=1)
        lse[i] = m + np.log(Z)
    return {"out": out, "weight_sum": wsum, "sink_weight": swgt, "lse": lse, "rows": rows}


# --------------------------------------------------------------------------
# Comparison metric used by the parity tests
# --------------------------------------------------------------------------

def error_metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    """max |got - ref| and sum|got - ref| / sum|ref| (the aggregate relative
    error; an elementwise mean of |d|/|ref| is dominated by outputs near 0)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    denom = np.abs(ref).sum()
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_rel": float(d.sum() / denom) if denom > 0 else float(d.sum()),
        "nonfinite": int((~np.isfinite(got)).sum()),
    }
