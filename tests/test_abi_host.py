"""The C ABI library on the host: it loads, exports every entry point that
include/smla.h declares, and its host-side argument checks return the
documented status codes before anything touches a GPU (no compute call)."""

import ctypes
import os
import sys
import re
import subprocess
from pathlib import Path

import pytest

import sparse_mla_attention_token_amd as smla

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "smla.h"


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"SMLA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_every_entry_point_the_binding_knows():
    assert declared_functions() == sorted(smla.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = smla.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(smla.LIB_PATH)], capture_output=True, text=True)
    exported = {ln.split()[-1] for ln in out.stdout.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported
    # nothing but the C ABI is exported
    assert exported == set(declared_functions())


def test_version_and_status_strings():
    assert smla.version() == 100
    assert smla.status_string(0) == "ok"
    assert "unsupported" in smla.status_string(3)
    assert smla.status_string(99) == "unknown status"


def good_dims(**kw):
    d = dict(q_or_T=4, H=128, topk=64, num_seqs=1, page_size=64, max_pages=4, num_pages=4)
    d.update(kw)
    return smla.make_dims(**d)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def call(dims, **ptrs):
    base = dict(out=FAKE, q=FAKE, kv_pages=FAKE, page_table=FAKE, cu_seqlens_q=FAKE, scales=None,
                indices=FAKE, topk_lengths=FAKE, sink=None)
    base.update(ptrs)
    return smla.call_raw(dims=dims, **base)


def test_null_dims():
    assert call(None) == 1


@pytest.mark.parametrize("field,value,code", [
    ("qk_depth", 512, 2), ("v_depth", 576, 2), ("num_tokens", -1, 2), ("topk", -3, 2),
    ("num_seqs", 0, 2), ("page_size", 0, 2), ("max_pages_per_seq", 0, 2), ("num_pages", 0, 2),
    ("num_heads", 0, 2), ("num_heads", 20, 3), ("num_heads", 144, 3), ("num_heads", 8, 3),
])
def test_shape_and_support_checks(field, value, code):
    d = good_dims()
    setattr(d, field, value)
    assert call(d) == code


def test_pool_above_4gib_passes_the_size_checks():
    # a misaligned q is reported only after the pool size was accepted
    d = good_dims(num_pages=131072, page_size=64)          # 8.4 M rows, 4.83 GB of latent rows
    assert call(d, q=FAKE + 4) == 4
    d = good_dims(num_pages=2_000_000, page_size=64)       # 73.7 GB
    assert call(d, q=FAKE + 4) == 4
    d = good_dims(num_pages=0x7FFFFFFF, page_size=2)       # 2^32 - 2 rows, the largest pool
    assert call(d, q=FAKE + 4) == 4


def test_pool_of_2_32_rows_or_more_is_unsupported():
    assert call(good_dims(num_pages=0x7FFFFFFF, page_size=3), q=FAKE + 4) == 3
    assert call(good_dims(num_pages=1 << 31, page_size=1), q=FAKE + 4) == 3   # more pages than an int holds


def test_scale_table_of_4gib_is_unsupported():
    # 60 M rows x 18 block scales x 4 B = 4.32 GB: rejected before any launch
    d = good_dims(num_pages=937_500, page_size=64)
    assert smla.call_raw(dims=d, out=FAKE, q=FAKE, kv_pages=FAKE, page_table=FAKE, cu_seqlens_q=FAKE,
                         scales=FAKE, indices=FAKE, topk_lengths=FAKE, sink=None, scale_block_size=32) == 3


@pytest.mark.parametrize("sbs,code", [(-1, 2), (40, 3), (8, 3)])
def test_scale_block_size_checks(sbs, code):
    assert smla.call_raw(dims=good_dims(), out=FAKE, q=FAKE, kv_pages=FAKE, page_table=FAKE,
                         cu_seqlens_q=FAKE, scales=FAKE, indices=FAKE, topk_lengths=FAKE, sink=None,
                         scale_block_size=sbs) == code


@pytest.mark.parametrize("missing", ["out", "q", "kv_pages", "page_table", "cu_seqlens_q", "indices",
                                     "topk_lengths"])
def test_null_pointers(missing):
    assert call(good_dims(), **{missing: None}) == 1


def test_scales_required_for_scaled_modes():
    assert smla.call_raw(dims=good_dims(), out=FAKE, q=FAKE, kv_pages=FAKE, page_table=FAKE,
                         cu_seqlens_q=FAKE, scales=None, indices=FAKE, topk_lengths=FAKE, sink=None,
                         scale_block_size=576) == 1


@pytest.mark.parametrize("which,addr", [("out", FAKE + 8), ("q", FAKE + 2), ("kv_pages", FAKE + 4),
                                         ("indices", FAKE + 2), ("sink", FAKE + 1)])
def test_misaligned_pointers(which, addr):
    assert call(good_dims(), **{which: addr}) == 4


def test_zero_tokens_is_a_no_op():
    assert call(good_dims(q_or_T=0), out=None, q=None, indices=None) == 0


@pytest.mark.parametrize("scale", [0.0, -0.5, float("inf"), float("nan")])
def test_softmax_scale_must_be_finite_and_positive(scale):
    assert smla.call_raw(dims=good_dims(), out=FAKE, q=FAKE, kv_pages=FAKE, page_table=FAKE,
                         cu_seqlens_q=FAKE, scales=None, indices=FAKE, topk_lengths=FAKE, sink=None,
                         scale=scale) == 2


# ---------------------------------------------------------------- split top-k entry points

def call_split(dims, num_splits, workspace=FAKE, workspace_bytes=1 << 40, **ptrs):
    base = dict(out=FAKE, q=FAKE, kv_pages=FAKE, page_table=FAKE, cu_seqlens_q=FAKE, scales=None,
                indices=FAKE, topk_lengths=FAKE, sink=None)
    base.update(ptrs)
    return smla.call_raw(dims=dims, num_splits=num_splits, workspace=workspace,
                         workspace_bytes=workspace_bytes, **base)


def test_split_workspace_size_is_the_partial_results():
    T, H, K = 7, 48, 300
    for S in (2, 3, 8):
        rows = T * S * H
        o = -(-rows * 512 * 4 // 256) * 256
        ml = -(-rows * 2 * 4 // 256) * 256
        assert smla.split_workspace_bytes(T, H, K, S) == o + ml
    assert smla.split_workspace_bytes(T, H, K, 1) == 0
    assert smla.split_workspace_bytes(T, H, K, 0) == 0


@pytest.mark.parametrize("T,H,K,sbs,expect", [
    (128, 128, 2048, 0, 1),      # decode: two 64-head groups per token fill the CUs in one run
    (64, 128, 2048, 0, 4),       # fewer tokens: 4 runs of the one-workgroup kernel
    (4096, 128, 2048, 0, 1),     # prefill fills the CUs already
    (16, 16, 64, 0, 1),          # one tile: nothing to split
    (2, 128, 2048, 0, 16),       # runs of 2 tiles
    (64, 128, 2048, 32, 4),      # blockwise: one workgroup per token (all heads), 4 runs
    (1, 128, 100000, 0, 64),     # capped
])
def test_auto_splits(T, H, K, sbs, expect):
    assert smla.auto_splits(T, H, K, sbs) == expect


@pytest.mark.parametrize("S", [0, -1, 65])
def test_split_count_out_of_range(S):
    assert call_split(good_dims(), S) == 2


def test_split_workspace_checks():
    need = smla.split_workspace_bytes(4, 128, 64, 2)
    assert call_split(good_dims(), 2, workspace=None) == 1
    assert call_split(good_dims(), 2, workspace=FAKE + 16) == 4
    assert call_split(good_dims(), 2, workspace_bytes=need - 1) == 2


def test_one_split_needs_no_workspace():
    # num_splits = 1 is sparse_mla_prefill: the workspace is not looked at
    assert call_split(good_dims(), 1, workspace=None, workspace_bytes=0, out=None) == 1   # still validates out


# ---------------------------------------------------------------- single-pass entry point

def call_single(dims, sbs=0, num_splits=1, **ptrs):
    base = dict(out=FAKE, q=FAKE, kv_pages=FAKE, page_table=FAKE, cu_seqlens_q=FAKE, scales=FAKE,
                indices=FAKE, topk_lengths=FAKE, sink=None)
    base.update(ptrs)
    return smla.call_raw(dims=dims, single_pass=True, num_splits=num_splits, scale_block_size=sbs,
                         workspace=FAKE, workspace_bytes=1 << 40, **base)


@pytest.mark.parametrize("sbs", [16, 32, 288, 560])
def test_single_pass_rejects_blockwise_scales(sbs):
    assert call_single(good_dims(), sbs=sbs) == 3


def test_single_pass_checks_like_the_split_entry():
    assert call_single(None) == 1
    assert call_single(good_dims(), out=None) == 1
    assert call_single(good_dims(), num_splits=65) == 2
    assert call_single(good_dims(), q=FAKE + 8) == 4
    assert call_single(good_dims(q_or_T=0)) == 0


# ---------------------------------------------------------------- indexer entry points

def index_dims(**kw):
    d = dict(T=4, H=64, num_seqs=1, page_size=64, max_pages=4, num_pages=4, score_stride=256, topk=64)
    d.update(kw)
    return smla.make_index_dims(**d)


def call_scores(dims, **ptrs):
    lib = smla.load_library()
    base = dict(scores=FAKE, q=FAKE, q_scale=FAKE, k_pages=FAKE, k_scale=FAKE, page_table=FAKE,
                cu_seqlens_q=FAKE, seq_lens_k=FAKE)
    base.update(ptrs)
    return lib.sparse_mla_index_scores(*base.values(), ctypes.byref(dims) if dims is not None else None, None)


def call_topk(dims, **ptrs):
    lib = smla.load_library()
    base = dict(indices=FAKE, topk_lengths=FAKE, scores=FAKE, cu_seqlens_q=FAKE, seq_lens_k=FAKE)
    base.update(ptrs)
    return lib.sparse_mla_index_topk(*base.values(), ctypes.byref(dims) if dims is not None else None, None)


def test_index_checks():
    assert call_scores(None) == 1 and call_topk(None) == 1
    d = index_dims()
    d.depth = 64
    assert call_scores(d) == 2 and call_topk(d) == 2
    for H in (48, 160):
        assert call_scores(index_dims(H=H)) == 3
    assert call_scores(index_dims(score_stride=0)) == 2
    assert call_scores(index_dims(topk=-1)) == 2
    assert call_scores(index_dims(num_pages=1 << 30)) == 3          # pool above 4 GiB
    assert call_scores(index_dims(), q_scale=None) == 1
    assert call_scores(index_dims(), q_scale=FAKE + 8) == 4          # read 16 bytes at a time
    assert call_scores(index_dims(), scores=FAKE + 2) == 4
    assert call_topk(index_dims(), topk_lengths=None) == 1
    assert call_scores(index_dims(T=0)) == 0 and call_topk(index_dims(T=0)) == 0


# ---------------------------------------------------------------- dense prefill

def dense_dims(**kw):
    d = dict(num_seqs=2, max_prompt_len=300, H=16, Hkv=16, page_size=64, max_pages=5, num_pages=10, causal=True)
    d.update(kw)
    return smla.make_dense_dims(**d)


def call_dense(dims, scale=0.1, sbs=0, **ptrs):
    lib = smla.load_library()
    base = dict(out=FAKE, q=FAKE, k_nope=FAKE, v=FAKE, k_rope=FAKE, k_rope_scales=None, page_table=FAKE,
                valid_length=FAKE)
    base.update(ptrs)
    return lib.mla_dense_prefill(*base.values(), ctypes.c_float(scale), sbs,
                                 ctypes.byref(dims) if dims is not None else None, None)


def test_dense_checks():
    # every call below fails a host check, so nothing is launched
    assert call_dense(None) == 1
    assert call_dense(dense_dims(H=16, Hkv=5)) == 2                 # kv heads must divide heads
    assert call_dense(dense_dims(max_pages=4)) == 2                 # 4 x 64 rows < 300
    d = dense_dims()
    d.causal = 2
    assert call_dense(d) == 2
    assert call_dense(dense_dims(num_seqs=0)) == 2
    d = dense_dims()
    d.v_depth = 512
    assert call_dense(d) == 3
    for sbs in (8, 20, -1):
        assert call_dense(dense_dims(), sbs=sbs, k_rope_scales=FAKE) == 3
    assert call_dense(dense_dims(), sbs=32) == 1                    # scales required
    assert call_dense(dense_dims(num_pages=1 << 20, Hkv=16, H=16)) == 3   # K_nope cache >= 2 GiB
    for scale in (0.0, -1.0, float("inf"), float("nan")):
        assert call_dense(dense_dims(), scale=scale) == 2
    assert call_dense(dense_dims(), q=None) == 1
    assert call_dense(dense_dims(), k_rope=FAKE + 8) == 4
    assert call_dense(dense_dims(), valid_length=FAKE + 2) == 4


def test_missing_library_raises_instead_of_falling_back(tmp_path):
    # a fresh process pointed at a library that does not exist: loading fails
    # loudly, there is no CPU path to fall back on
    code = ("import sparse_mla_attention_token_amd as s\n"
            "try:\n    s.load_library()\nexcept ImportError as e:\n    print('raised', e)\n")
    env = dict(os.environ, SMLA_LIB=str(tmp_path / "absent.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=str(Path(__file__).resolve().parents[1]), timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("raised"), r.stdout + r.stderr


def test_product_code_never_imports_the_oracle():
    pkg = Path(__file__).resolve().parents[1] / "sparse_mla_attention_token_amd"
    for f in pkg.rglob("*.py"):
        text = f.read_text()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f


# ---------------------------------------------------------------- binding-side tensor checks
#
# The library sizes every buffer from the dims it is given, so the binding
# rejects a tensor of the wrong device, dtype or shape with ValueError before
# any pointer reaches the C ABI.  Checked here on host tensors (allow_cpu
# turns off only the "must be on a GPU" rule).

def _prefill_args(sbs=32, sink=True):
    import workloads as W

    s = W.CaseSpec(name="chk", num_seqs=2, q_per_seq=3, ctx=130, q_pos0=127, num_heads=32, topk=64,
                   page_size=16, shuffle_pages=True, scale_block_size=sbs, sink=sink)
    c = W.make_case(s, seed=5)
    return dict(q=c.q, kv_pages=c.kv_pages, page_table=c.page_table, cu_seqlens_q=c.cu_seqlens_q,
                indices=c.indices, topk_lengths=c.topk_lengths, scale_block_size=sbs, scales=c.scales,
                sink=c.sink)


def test_prefill_validation_accepts_the_workload_tensors():
    import torch

    for sbs, sink in ((0, False), (576, True), (32, True), (16, False)):
        a = _prefill_args(sbs, sink)
        T, H = a["q"].shape[:2]
        smla.validate_prefill_args(**a, out=torch.empty((T, H, 512), dtype=torch.bfloat16), allow_cpu=True)


def test_prefill_rejects_host_tensors_without_touching_the_library():
    with pytest.raises(ValueError, match="GPU"):
        smla.sparse_mla_prefill(scale=0.1, **_prefill_args())


@pytest.mark.parametrize("what", ["scales_cols", "scales_rows", "scales_missing", "sink_dtype", "sink_len",
                                  "out_small", "out_dtype", "cu_short", "indices_rows", "lengths_dtype",
                                  "q_depth", "q_dtype", "kv_width", "pt_dtype", "noncontig", "neg_sbs"])
def test_prefill_rejects_mismatched_tensors(what):
    import torch

    a = _prefill_args()
    T, H = a["q"].shape[:2]
    out = None
    if what == "scales_cols":
        a["scales"] = a["scales"][:, :1].contiguous()          # [rows, 1] with sbs = 32
    elif what == "scales_rows":
        a["scales"] = a["scales"][:-16].contiguous()
    elif what == "scales_missing":
        a["scales"] = None
    elif what == "sink_dtype":
        a["sink"] = a["sink"].to(torch.bfloat16)
    elif what == "sink_len":
        a["sink"] = a["sink"][:-1].contiguous()
    elif what == "out_small":
        out = torch.empty((T, H - 16, 512), dtype=torch.bfloat16)
    elif what == "out_dtype":
        out = torch.empty((T, H, 512), dtype=torch.float32)
    elif what == "cu_short":
        a["cu_seqlens_q"] = a["cu_seqlens_q"][:-1].contiguous()
    elif what == "indices_rows":
        a["indices"] = a["indices"][:-1].contiguous()
    elif what == "lengths_dtype":
        a["topk_lengths"] = a["topk_lengths"].to(torch.int64)
    elif what == "q_depth":
        a["q"] = a["q"][:, :, :512].contiguous()
    elif what == "q_dtype":
        a["q"] = a["q"].float()
    elif what == "kv_width":
        a["kv_pages"] = a["kv_pages"][:, :, :512].contiguous()
    elif what == "pt_dtype":
        a["page_table"] = a["page_table"].to(torch.int64)
    elif what == "noncontig":
        a["indices"] = a["indices"].t().contiguous().t()
    elif what == "neg_sbs":
        a["scale_block_size"] = -32
    with pytest.raises(ValueError):
        smla.validate_prefill_args(**a, out=out, allow_cpu=True)


def test_index_validation():
    import torch
    import workloads as W

    spec = W.INDEXER_CONFIGS["indexer_tiny"]
    c = W.make_indexer_case(spec, W.INDEXER_SEEDS["indexer_tiny"], device="cpu")
    base = dict(q=c.q, q_scale=c.q_scale, k_pages=c.k_pages, k_scale=c.k_scale, page_table=c.page_table,
                cu_seqlens_q=c.cu_seqlens_q, seq_lens_k=c.seq_lens_k, score_stride=spec.stride)
    smla.validate_index_scores_args(**base, allow_cpu=True)
    for key, bad in (("q_scale", c.q_scale[:, :-1].contiguous()), ("k_scale", c.k_scale[:-1].contiguous()),
                     ("q", c.q[:, :, :64].contiguous()), ("seq_lens_k", c.seq_lens_k.to(torch.int64)),
                     ("cu_seqlens_q", c.cu_seqlens_q[:-1].contiguous())):
        with pytest.raises(ValueError):
            smla.validate_index_scores_args(**dict(base, **{key: bad}), allow_cpu=True)
    with pytest.raises(ValueError):
        smla.validate_index_scores_args(**base, scores=torch.empty((spec.num_tokens, spec.stride - 1)),
                                        allow_cpu=True)
    scores = torch.zeros((spec.num_tokens, spec.stride))
    smla.validate_index_topk_args(scores, c.cu_seqlens_q, c.seq_lens_k, spec.topk, allow_cpu=True)
    with pytest.raises(ValueError):
        smla.validate_index_topk_args(scores, c.cu_seqlens_q, c.seq_lens_k, spec.topk,
                                      indices=torch.empty((spec.num_tokens, spec.topk - 1), dtype=torch.int32),
                                      allow_cpu=True)
    with pytest.raises(ValueError):
        smla.validate_index_topk_args(scores.double(), c.cu_seqlens_q, c.seq_lens_k, spec.topk, allow_cpu=True)
    with pytest.raises(ValueError, match="GPU"):
        smla.sparse_mla_index_scores(**base)


def test_dense_validation():
    import torch
    import workloads as W

    spec = W.DENSE_CONFIGS["dense_tiny"]
    c = W.make_dense_case(spec, W.DENSE_SEEDS["dense_tiny"], device="cpu")
    base = dict(q=c.q, k_nope=c.k_nope, v=c.v, k_rope=c.k_rope, k_rope_scales=c.k_rope_scales,
                page_table=c.page_table, valid_length=c.valid_length, scale_block_size=spec.scale_block_size,
                max_prompt_len=spec.max_prompt_len)
    smla.validate_dense_args(**base, allow_cpu=True)
    bads = [("k_rope_scales", None), ("k_rope", c.k_rope[:, :, :32].contiguous()),
            ("q", c.q[:-1].contiguous()), ("valid_length", c.valid_length[:-1].contiguous()),
            ("v", c.v.float())]
    if c.k_rope_scales is not None:
        bads.append(("k_rope_scales", c.k_rope_scales[:-1].contiguous()))
    for key, bad in bads:
        if key == "k_rope_scales" and spec.scale_block_size == 0:
            continue
        with pytest.raises(ValueError):
            smla.validate_dense_args(**dict(base, **{key: bad}), allow_cpu=True)
    with pytest.raises(ValueError, match="GPU"):
        smla.mla_dense_prefill(scale=0.1, scale_block_size=spec.scale_block_size, **{
            k: v for k, v in base.items() if k != "scale_block_size"})


# ---------------------------------------------------------------- no-allocation entry point

def test_noalloc_checks_run_before_any_device_call():
    d = good_dims()
    assert smla.call_raw(dims=None, out=FAKE, q=FAKE, kv_pages=FAKE, page_table=FAKE, cu_seqlens_q=FAKE,
                         indices=FAKE, topk_lengths=FAKE, noalloc=True, num_splits=2) == 1
    assert call(d, q=None, noalloc=True, num_splits=2) == 1
    assert call(d, noalloc=True, num_splits=0) == 2
    assert call(d, noalloc=True, num_splits=65) == 2
    assert call(d, q=FAKE + 4, noalloc=True, num_splits=2) == 4


def test_noalloc_rejects_partials_beyond_the_scratch_array():
    cap = smla.noalloc_scratch_bytes()
    assert cap == 80 << 20
    big = good_dims(q_or_T=4096, H=128, topk=2048)
    assert smla.split_workspace_bytes(4096, 128, 2048, 8) > cap
    assert call(big, noalloc=True, num_splits=8) == 6
    assert "scratch" in smla.status_string(6)
    # the largest run count that fits 128 tokens x 128 heads is 2
    assert smla.split_workspace_bytes(128, 128, 2048, 2) <= cap < smla.split_workspace_bytes(128, 128, 2048, 3)
    assert call(good_dims(q_or_T=128, H=128, topk=2048), noalloc=True, num_splits=3) == 6


def test_probe_library_exports_its_header():
    from sparse_mla_attention_token_amd import probe

    text = (ROOT / "include" / "smla_probe.h").read_text()
    declared = sorted(set(re.findall(r"SMLA_PROBE_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))
    assert declared == sorted(probe.PROBE_SYMBOLS)
    lib = probe.load_probe_library()
    out = subprocess.run(["nm", "-D", "--defined-only", str(probe.PROBE_LIB_PATH)], capture_output=True, text=True)
    exported = {ln.split()[-1] for ln in out.stdout.splitlines() if " T " in ln}
    assert exported == set(declared)
    # host-side checks and the FLOP count, no launch
    assert lib.smla_probe_mfma(7, 1, 1, None, None) == 1
    assert lib.smla_probe_mfma_flop(0, 10, 2) == 2 * 4 * 10 * 4 * (2 * 32 * 32 * 64)
    assert lib.smla_probe_mfma_flop(1, 10, 2) == 2 * 4 * 10 * 4 * (2 * 32 * 32 * 16)
    assert lib.smla_probe_gather(None, 0, None, 1, 1, None, None) == 1
    assert lib.smla_probe_coexec(3, 0, 1, 1, None, None, None) == 1
    assert lib.smla_probe_coexec(0, 5, 1, 1, None, None, None) == 1
