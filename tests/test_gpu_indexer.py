"""GPU parity of the FP8 lightning indexer and its top-k stage (through the C ABI).

Scores: the FP8 products are exact in f32 and the matrix cores sum each
64-deep block with about 14 significant bits, so per head the dot product is
within 2^-13 of sum_c |q_c k_c|; the relu, weights and head sum add f32
rounding.  The bar, with a factor 8 of margin:
    |gpu - oracle| <= 2^-10 * k_scale * sum_h |q_scale_h| * sum_c |q_hc k_c|
and -inf exactly where the oracle has -inf.
Top-k: bit-exact against the oracle's selection applied to the GPU's own f32
scores (the selection is decided in the kernel's precision on both sides).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_token_amd as smla
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    smla.load_library()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_scores(g, stride):
    s = smla.sparse_mla_index_scores(g.q, g.q_scale, g.k_pages, g.k_scale, g.page_table, g.cu_seqlens_q,
                                     g.seq_lens_k, stride)
    torch.cuda.synchronize()
    return s


def magnitude(a, tokens, stride):
    """k_scale * sum_h |q_scale| * sum_c |q k| per (token, key) (the error scale)."""
    P = a["k_pages"].shape[1]
    flat = a["k_pages"].reshape(-1, 128)
    cu = a["cu_seqlens_q"]
    n_t = oracle.causal_counts(cu, a["seq_lens_k"])
    out = np.zeros((len(tokens), stride))
    for i, t in enumerate(tokens):
        b = int(np.searchsorted(cu, t, side="right") - 1)
        n = int(min(n_t[t], stride))
        if n == 0:
            continue
        rows = oracle.key_rows(b, n, a["page_table"], P, a["k_pages"].shape[0])
        r = np.where(rows >= 0, rows, 0)
        k = np.abs(oracle.decode_e4m3fn(flat[r]))
        q = np.abs(oracle.decode_e4m3fn(a["q_codes"][t]))
        out[i, :n] = (np.abs(a["q_scale"][t].astype(np.float64)) @ (q @ k.T)) * a["k_scale"][r]
    return out


def check_scores(got, a, tokens, stride, label):
    ref = oracle.indexer_scores(**a, score_stride=stride, tokens=tokens)
    got = got.double().cpu().numpy()
    fin = np.isfinite(ref)
    assert (np.isneginf(got) == np.isneginf(ref)).all(), f"{label}: -inf pattern differs"
    assert np.isfinite(got[fin]).all(), label
    bound = 2.0 ** -10 * magnitude(a, tokens, stride) + 1e-30
    err = np.abs(got[fin] - ref[fin])
    worst = float((err / bound[fin]).max()) if fin.any() else 0.0
    say(f"  {label}: {fin.sum()} scores, max err / bound = {worst:.3e}, max err = {err.max() if fin.any() else 0:.3e}")
    assert worst <= 1.0, label


def check_topk(scores, g, K, label):
    idx, lens = smla.sparse_mla_index_topk(scores, g.cu_seqlens_q, g.seq_lens_k, K)
    torch.cuda.synchronize()
    n_t = oracle.causal_counts(g.cu_seqlens_q.cpu().numpy(), g.seq_lens_k.cpu().numpy())
    n_valid = np.minimum(n_t, scores.shape[1])
    ref_idx, ref_len = oracle.topk_select(scores.cpu().numpy(), n_valid, K)
    got_idx = idx.cpu().numpy().view(np.uint32)
    got_len = lens.cpu().numpy().view(np.uint32)
    say(f"  {label}: top-{K}, lengths {got_len.min()}..{got_len.max()}")
    assert np.array_equal(got_len, ref_len), label
    assert np.array_equal(got_idx, ref_idx), label
    return idx, lens


def case_of(spec, seed, q_lens=None):
    c = W.make_indexer_case(spec, seed, device="cpu", q_lens=q_lens)
    return c, c.host_arrays(), c.to("cuda")


def test_tiny_scores_and_topk():
    spec = W.INDEXER_CONFIGS["indexer_tiny"]
    say(f"case {spec}")
    c, a, g = case_of(spec, W.INDEXER_SEEDS["indexer_tiny"])
    s = gpu_scores(g, spec.stride)
    check_scores(s, a, np.arange(spec.num_tokens), spec.stride, "tiny")
    check_topk(s, g, spec.topk, "tiny")


@pytest.mark.parametrize("H", [32, 64, 96, 128])
@pytest.mark.parametrize("P", [1, 16, 64])
def test_heads_and_page_sizes(H, P):
    spec = W.IndexerSpec("ix", num_seqs=2, q_per_seq=9, ctx=300, num_heads=H, page_size=P, topk=100,
                         shuffle_pages=True, spare_pages=2)
    say(f"case H={H} P={P}")
    c, a, g = case_of(spec, 2100 + H + P)
    s = gpu_scores(g, spec.stride)
    check_scores(s, a, np.arange(spec.num_tokens), spec.stride, f"H{H}/P{P}")
    check_topk(s, g, spec.topk, f"H{H}/P{P}")


def test_ragged_sequences_and_edge_cases():
    # query counts 5, 0, 7, 1, 6 over key counts 70, 9, 3, 130, 200: an empty
    # sequence, more queries than keys (leading queries see nothing), a
    # workgroup's four tokens spanning sequences, a stride wider than any
    # sequence, and one page id out of range
    spec = W.IndexerSpec("ragged", num_seqs=5, q_per_seq=0, ctx=200, num_heads=64, page_size=16, topk=48,
                         shuffle_pages=True, score_stride=256)
    say("case ragged")
    c, a, g = case_of(spec, 2201, q_lens=[5, 0, 7, 1, 6])
    lk = np.array([70, 9, 3, 130, 200], dtype=np.int32)
    a["seq_lens_k"] = lk
    g.seq_lens_k.copy_(torch.from_numpy(lk))
    a["page_table"] = a["page_table"].copy()
    a["page_table"][4, 3] = 10 ** 6
    g.page_table.copy_(torch.from_numpy(a["page_table"]))
    s = gpu_scores(g, spec.stride)
    check_scores(s, a, np.arange(int(a["cu_seqlens_q"][-1])), spec.stride, "ragged")
    idx, lens = check_topk(s, g, spec.topk, "ragged")
    assert (lens.cpu().numpy()[5:8] == [0, 0, 0]).all()   # 7 queries over 3 keys: positions -4..2


def test_topk_ties_and_small_rows():
    # scores written by hand: heavy ties, rows shorter than K, K = 1
    T, stride = 6, 700
    rng = np.random.default_rng(11)
    sc = np.round(rng.normal(size=(T, stride)), 1).astype(np.float32)
    sc[2, :] = 0.0
    sc[3, ::2] = -0.0
    sc[4, 5] = np.nan
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    lk = torch.tensor([stride], dtype=torch.int32, device="cuda")   # positions 694..699
    g = type("G", (), {"cu_seqlens_q": cu, "seq_lens_k": lk})()
    s = torch.from_numpy(sc).cuda()
    for K in (1, 64, 695, 699, 700, 900):
        check_topk(s, g, K, f"ties K={K}")


@pytest.mark.parametrize("stride", [1000, 5000, 12000, 20000])
def test_topk_row_lengths(stride):
    # rows held in registers (up to 4, 16 or 32 keys per thread) and rows
    # re-read from memory (longer than 16384)
    T = 4
    rng = np.random.default_rng(stride)
    sc = np.round(rng.normal(size=(T, stride)) * 8).astype(np.float32)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    lk = torch.tensor([stride], dtype=torch.int32, device="cuda")
    g = type("G", (), {"cu_seqlens_q": cu, "seq_lens_k": lk})()
    s = torch.from_numpy(sc).cuda()
    for K in (7, stride // 3, stride - 2):
        check_topk(s, g, K, f"stride {stride} K={K}")


def test_end_to_end_indexer_topk_attention():
    # indices from the GPU indexer drive the GPU attention; the attention is
    # checked against its oracle on the same index lists
    aspec = W.CaseSpec("e2e", num_seqs=2, q_per_seq=6, ctx=512, q_pos0=506, num_heads=64, topk=128,
                       page_size=64, shuffle_pages=True, lengths="full")
    ispec = W.IndexerSpec("e2e", num_seqs=2, q_per_seq=6, ctx=512, num_heads=64, topk=128, page_size=64,
                          shuffle_pages=True)
    say("case end to end")
    att = W.make_case(aspec, seed=2301, device="cpu")
    c, a, g = case_of(ispec, 2302)
    s = gpu_scores(g, ispec.stride)
    idx, lens = check_topk(s, g, ispec.topk, "e2e")
    ag = att.to("cuda")
    out = smla.sparse_mla_prefill(ag.q, ag.kv_pages, ag.page_table, ag.cu_seqlens_q, idx.contiguous(), lens,
                                  ag.scale, 0, None, None)
    torch.cuda.synchronize()
    h = att.host_arrays()
    h["indices"] = idx.cpu().numpy().view(np.uint32)
    h["topk_lengths"] = lens.cpu().numpy().view(np.uint32)
    ref = oracle.sparse_mla_prefill(h["q_bits"], h["kv_pages"], h["page_table"], h["cu_seqlens_q"], h["scales"],
                                    h["indices"], h["topk_lengths"], h["sink"], h["scale"], h["scale_block_size"])
    m = oracle.error_metrics(out.float().cpu().double().numpy(), ref["out"])
    say(f"  e2e attention: max_abs={m['max_abs']:.3e} mean_rel={m['mean_rel']:.3e}")
    assert m["nonfinite"] == 0 and m["max_abs"] <= 2e-2 and m["mean_rel"] <= 5e-3


def test_dsv32_indexer_full_size_sampled():
    spec = W.INDEXER_CONFIGS["indexer_dsv32"]
    say(f"case {spec.name} full size")
    g = W.make_indexer_case(spec, W.INDEXER_SEEDS["indexer_dsv32"], device="cuda")
    s = gpu_scores(g, spec.stride)
    tokens = np.array([0, 1, 777, 2048, 3001, 4095])
    a = {k: v for k, v in g.to("cpu").host_arrays().items()}
    check_scores(s[torch.from_numpy(tokens).cuda()], a, tokens, spec.stride, "indexer_dsv32")
    idx, lens = smla.sparse_mla_index_topk(s, g.cu_seqlens_q, g.seq_lens_k, spec.topk)
    torch.cuda.synchronize()
    n_t = oracle.causal_counts(a["cu_seqlens_q"], a["seq_lens_k"])
    ref_idx, ref_len = oracle.topk_select(s[torch.from_numpy(tokens).cuda()].cpu().numpy(), n_t[tokens], spec.topk)
    assert np.array_equal(lens.cpu().numpy().view(np.uint32)[tokens], ref_len)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32)[tokens], ref_idx)
