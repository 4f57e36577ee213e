"""Pins of the CPU float64 oracle against things other than itself.

Every check here fixes some part of the oracle with an independent route:
torch's own FP8 / bf16 casts, an unpaged copy of the cache, torch's
scaled-dot-product attention in float64 (a library routine), closed forms of
special cases, and invariants that hold for any correct implementation.
Sources: the Modular pages "mla_sm100_prefill_sparse_fp8" (arguments, scale
modes, sink, BF16 q/out, FP8 e4m3fn cache) and "mla_prefill_sparse_qkv_fp8"
(V is the first 512 columns of the gathered latent).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_spec(**kw):
    base = dict(name="pin", num_seqs=2, q_per_seq=5, ctx=96, q_pos0=91, num_heads=4, topk=96,
                page_size=16, shuffle_pages=True)
    base.update(kw)
    return W.CaseSpec(**base)


def run_oracle(case, tokens=None, **over):
    a = case.host_arrays()
    a.update(over)
    return oracle.sparse_mla_prefill(a["q_bits"], a["kv_pages"], a["page_table"], a["cu_seqlens_q"],
                                     a["scales"], a["indices"], a["topk_lengths"], a["sink"], a["scale"],
                                     a["scale_block_size"], tokens=tokens)


# ---------------------------------------------------------------- formats

def test_e4m3fn_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_m, nan_r = np.isnan(mine), np.isnan(ref)
    assert (nan_m == nan_r).all()
    assert nan_m.sum() == 2                      # 0x7F and 0xFF
    assert (mine[~nan_m] == ref[~nan_r]).all()
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


def test_bf16_decoder_matches_torch_on_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan_m, nan_r = np.isnan(mine), np.isnan(ref)
    assert (nan_m == nan_r).all()
    assert (mine[~nan_m] == ref[~nan_r]).all()


# ---------------------------------------------------------------- paging

def unpaged_sequences(case):
    """Each sequence's latent rows in logical order: its pages concatenated
    in page-table order (an independent route to the paged lookup)."""
    kv = case.kv_pages.numpy()
    pt = case.page_table.numpy()
    return [np.concatenate([kv[p] for p in pt[b]], axis=0) for b in range(case.spec.num_seqs)]


def test_gather_matches_unpaged_copy():
    case = W.make_case(small_spec(lengths="uniform:1:96", topk=80), seed=7)
    a = case.host_arrays()
    rows = oracle.translate_rows(a["indices"], a["topk_lengths"], a["page_table"], a["cu_seqlens_q"],
                                 case.spec.page_size, case.spec.num_pages)
    got = oracle.gather_rows(a["kv_pages"], rows)
    seqs = unpaged_sequences(case)
    T, K = a["indices"].shape
    for t in range(T):
        b = t // case.spec.q_per_seq
        L = min(int(a["topk_lengths"][t]), K)
        for j in range(K):
            if j < L:
                assert (got[t, j] == seqs[b][a["indices"][t, j]]).all()
            else:
                assert (got[t, j] == 0).all() and rows[t, j] == -1


def test_out_of_range_slots_are_masked():
    case = W.make_case(small_spec(topk=8, lengths="full", q_pos0=40), seed=3)
    a = case.host_arrays()
    base = run_oracle(case)
    idx = a["indices"].copy()
    pt = a["page_table"].copy()
    # slot 0 of token 0 beyond the page-table row, slot 1 of token 1 on a bad page id
    idx2 = np.concatenate([idx, np.zeros((idx.shape[0], 1), np.uint32)], axis=1)
    idx2[0, -1] = 10 ** 9
    L2 = a["topk_lengths"] + 1
    bad = run_oracle(case, indices=idx2, topk_lengths=L2)
    assert np.allclose(bad["out"][0], base["out"][0], rtol=0, atol=1e-13)
    pt2 = pt.copy()
    pt2[0, idx[1, 1] // case.spec.page_size] = -5
    masked = run_oracle(case, page_table=pt2)
    keep = np.delete(idx[1], 1)
    ref = run_oracle(case, indices=np.stack([np.concatenate([keep, [0]]).astype(np.uint32)] * idx.shape[0]),
                     topk_lengths=np.full(idx.shape[0], len(keep), np.uint32), page_table=pt2, tokens=[1])
    assert np.allclose(masked["out"][1], ref["out"][0], rtol=0, atol=1e-13)


def test_lengths_above_topk_are_clamped_and_empty_gives_zero():
    case = W.make_case(small_spec(topk=16, lengths="full", q_pos0=40, sink=True), seed=5)
    a = case.host_arrays()
    base = run_oracle(case)
    big = run_oracle(case, topk_lengths=np.full_like(a["topk_lengths"], 1000))
    assert np.array_equal(base["out"], big["out"])
    empty = run_oracle(case, topk_lengths=np.zeros_like(a["topk_lengths"]))
    assert (empty["out"] == 0).all()
    empty_nosink = run_oracle(case, topk_lengths=np.zeros_like(a["topk_lengths"]), sink=None)
    assert (empty_nosink["out"] == 0).all()


# ---------------------------------------------------------------- attention

def dense_reference(case, with_sink):
    """Dense causal attention over each sequence's whole prefix with torch SDPA
    in float64 on the unpaged, dequantised cache."""
    spec = case.spec
    seqs = unpaged_sequences(case)
    pt = case.page_table.numpy()
    outs = []
    for b in range(spec.num_seqs):
        codes = torch.from_numpy(seqs[b][: spec.ctx]).view(torch.float8_e4m3fn).to(torch.float64)
        if spec.scale_block_size:
            sc = case.scales.to(torch.float64).reshape(spec.num_pages, spec.page_size, -1)
            rows_sc = torch.cat([sc[p] for p in pt[b]], dim=0)[: spec.ctx]
            if rows_sc.shape[1] == 1:
                codes = codes * rows_sc
            else:
                codes = codes * rows_sc.repeat_interleave(spec.scale_block_size, dim=1)[:, : W.QK_DEPTH]
        k = codes
        v = codes[:, : W.V_DEPTH]
        q = case.q[b * spec.q_per_seq:(b + 1) * spec.q_per_seq].to(torch.float64).transpose(0, 1)  # [H, Tq, D]
        pos = case.positions[b * spec.q_per_seq:(b + 1) * spec.q_per_seq]
        allowed = torch.arange(spec.ctx)[None, :] <= pos[:, None]                                   # [Tq, S]
        H = spec.num_heads
        mask = torch.where(allowed, 0.0, -math.inf).to(torch.float64).expand(H, -1, -1)
        kk = k.expand(H, -1, -1)
        vv = v.expand(H, -1, -1)
        if with_sink:
            sink = case.sink.to(torch.float64)
            kk = torch.cat([kk, torch.zeros(H, 1, W.QK_DEPTH, dtype=torch.float64)], dim=1)
            vv = torch.cat([vv, torch.zeros(H, 1, W.V_DEPTH, dtype=torch.float64)], dim=1)
            extra = sink[:, None, None].expand(H, mask.shape[1], 1)
            mask = torch.cat([mask, extra], dim=2)
        o = F.scaled_dot_product_attention(q, kk.contiguous(), vv.contiguous(), attn_mask=mask.contiguous(),
                                           scale=case.scale)
        outs.append(o.transpose(0, 1))
    return torch.cat(outs, dim=0).numpy()


@pytest.mark.parametrize("sbs,sink", [(0, False), (0, True), (576, True), (32, False), (48, True)])
def test_whole_prefix_equals_dense_causal_sdpa(sbs, sink):
    spec = small_spec(scale_block_size=sbs, sink=sink, lengths="causal")
    case = W.make_case(spec, seed=11 + sbs)
    got = run_oracle(case)["out"]
    ref = dense_reference(case, with_sink=sink)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_weights_sum_to_one_minus_sink_mass():
    case = W.make_case(small_spec(sink=True, scale_block_size=576, lengths="uniform:1:96"), seed=21)
    r = run_oracle(case)
    assert np.allclose(r["weight_sum"] + r["sink_weight"], 1.0, rtol=0, atol=1e-12)
    assert (r["sink_weight"] > 0).all()
    r0 = run_oracle(case, sink=None)
    assert np.allclose(r0["weight_sum"], 1.0, rtol=0, atol=1e-12)


def test_sink_closed_form_and_limit():
    case = W.make_case(small_spec(sink=True), seed=23)
    with_sink = run_oracle(case)
    without = run_oracle(case, sink=None)
    # sink adds exp(sink) to the denominator only: out scales by (1 - p_sink)
    scaled = without["out"] * (1.0 - with_sink["sink_weight"])[:, :, None]
    assert np.allclose(with_sink["out"], scaled, rtol=1e-11, atol=1e-13)
    very_negative = run_oracle(case, sink=np.full(case.spec.num_heads, -1e4, np.float32))
    assert np.allclose(very_negative["out"], without["out"], rtol=0, atol=1e-15)


def test_topk_one_returns_the_dequantised_row():
    for sbs in (0, 576, 32):
        case = W.make_case(small_spec(scale_block_size=sbs, topk=4, lengths="full", q_pos0=40), seed=31)
        a = case.host_arrays()
        r = run_oracle(case, topk_lengths=np.ones_like(a["topk_lengths"]))
        seqs = unpaged_sequences(case)
        for t in range(a["indices"].shape[0]):
            b = t // case.spec.q_per_seq
            idx = a["indices"][t, 0]
            row = torch.from_numpy(seqs[b][idx][: W.V_DEPTH].copy()).view(torch.float8_e4m3fn).to(torch.float64)
            if sbs:
                phys = r["rows"][t, 0]
                s = case.scales[phys].to(torch.float64)
                row = row * (s[0] if s.numel() == 1 else s.repeat_interleave(sbs)[: W.V_DEPTH])
            assert np.array_equal(r["out"][t], np.broadcast_to(row.numpy(), r["out"][t].shape))


def test_zero_query_gives_mean_of_values():
    case = W.make_case(small_spec(lengths="uniform:1:96"), seed=41)
    a = case.host_arrays()
    zero_q = np.zeros_like(a["q_bits"])
    r = run_oracle(case, q_bits=zero_q)
    rows = r["rows"]
    flat = a["kv_pages"].reshape(-1, W.QK_DEPTH)
    for t in range(rows.shape[0]):
        valid = rows[t][rows[t] >= 0]
        vals = torch.from_numpy(flat[valid][:, : W.V_DEPTH].copy()).view(torch.float8_e4m3fn).to(torch.float64)
        mean = vals.mean(dim=0).numpy()
        assert np.allclose(r["out"][t], mean[None, :], rtol=1e-12, atol=1e-14)


def test_slot_permutation_invariance():
    case = W.make_case(small_spec(scale_block_size=32, sink=True, lengths="uniform:1:96"), seed=43)
    a = case.host_arrays()
    base = run_oracle(case)
    rng = np.random.default_rng(0)
    idx = a["indices"].copy()
    for t in range(idx.shape[0]):
        L = int(a["topk_lengths"][t])
        idx[t, :L] = idx[t, rng.permutation(L)]
    perm = run_oracle(case, indices=idx)
    assert np.allclose(perm["out"], base["out"], rtol=1e-12, atol=1e-14)


def test_scale_mode_equivalences():
    case = W.make_case(small_spec(lengths="uniform:1:96"), seed=47)
    a = case.host_arrays()
    rows = case.spec.num_pages * case.spec.page_size
    unit = run_oracle(case)
    ones = run_oracle(case, scales=np.ones((rows, 1), np.float32), scale_block_size=576)
    assert np.array_equal(unit["out"], ones["out"])
    c = np.exp2(np.random.default_rng(1).uniform(-3, 2, size=(rows, 1))).astype(np.float32)
    tw = run_oracle(case, scales=c, scale_block_size=576)
    tw_big = run_oracle(case, scales=c, scale_block_size=4096)
    assert np.array_equal(tw["out"], tw_big["out"])
    bw = run_oracle(case, scales=np.repeat(c, 18, axis=1), scale_block_size=32)
    assert np.allclose(bw["out"], tw["out"], rtol=1e-13, atol=1e-15)


def test_golden_two_key_example():
    """Hand-derived fixture (tests/golden/two_keys.json): the closed-form
    softmax of two logits, with and without a sink logit."""
    g = json.load(open(os.path.join(GOLDEN, "two_keys.json")))
    D = W.QK_DEPTH

    def dense(sparse):
        v = np.zeros(D)
        for c, x in sparse.items():
            if int(c) < D:
                v[int(c)] = x
        return v

    q, k0, k1 = dense(g["q"]), dense(g["k0"]), dense(g["k1"])
    qt = torch.from_numpy(q).to(torch.bfloat16).reshape(1, 1, D)
    kv = torch.from_numpy(np.stack([k0, k1])).to(torch.float8_e4m3fn).view(torch.uint8).reshape(1, 2, D)
    s0, s1 = g["scale"] * float(q @ k0), g["scale"] * float(q @ k1)
    for case in g["cases"]:
        z = case["sink"]
        if z is None:
            p1 = 1.0 / (1.0 + math.exp(s0 - s1))
            p0 = 1.0 - p1
        else:
            den = math.exp(s0) + math.exp(s1) + math.exp(z)
            p0, p1 = math.exp(s0) / den, math.exp(s1) / den
        res = oracle.sparse_mla_prefill(qt.view(torch.int16).numpy().view(np.uint16), kv.numpy(),
                                        np.array([[0]], np.int32), np.array([0, 1], np.int32), None,
                                        np.array([[0, 1]], np.uint32), np.array([2], np.uint32),
                                        None if z is None else np.array([z], np.float32), g["scale"], 0)
        out = res["out"][0, 0]
        for c in g["check_columns"]:
            assert abs(out[c] - (p0 * k0[c] + p1 * k1[c])) < 1e-12, (z, c)
        assert abs(res["weight_sum"][0, 0] - (p0 + p1)) < 1e-12


# ---------------------------------------------------------------- the comparison metric

def test_error_metrics_on_hand_values():
    """The metric every parity verdict rests on, fixed on values worked by hand:
    max_abs = max |got - ref|; mean_rel = sum |got - ref| / sum |ref| (the
    aggregate reading of the north-star's "mean relative error")."""
    m = oracle.error_metrics(np.array([1.0, 2.0, 4.0]), np.array([1.0, 1.0, 2.0]))
    # |d| = [0, 1, 2]: max 2, sum 3; sum |ref| = 4
    assert m["max_abs"] == 2.0
    assert m["mean_rel"] == 0.75
    assert m["nonfinite"] == 0
    # not the per-element mean of |d| / |ref| (= 2/3) nor sum|d| / sum|got| (= 3/7)
    m = oracle.error_metrics(np.array([[-1.0, 0.5], [3.0, -2.0]]), np.array([[1.0, 0.5], [2.0, -4.0]]))
    # |d| = [2, 0, 1, 2]: max 2, sum 5; sum |ref| = 7.5 (signs do not cancel)
    assert m["max_abs"] == 2.0
    assert abs(m["mean_rel"] - 5.0 / 7.5) < 1e-15


def test_error_metrics_counts_nonfinite_outputs():
    got = np.array([np.nan, 1.0, np.inf, -np.inf, 2.0])
    m = oracle.error_metrics(got, np.ones(5))
    assert m["nonfinite"] == 3
    # a NaN never passes a "<= bound" test, so the bound checks fail as well
    assert not (m["max_abs"] <= 2e-2)


def test_error_metrics_zero_reference_and_empty():
    # an all-zero reference (every slot masked, no sink): the sum of |d| itself
    m = oracle.error_metrics(np.array([0.5, -0.25, 0.0]), np.zeros(3))
    assert m["max_abs"] == 0.5 and m["mean_rel"] == 0.75 and m["nonfinite"] == 0
    m = oracle.error_metrics(np.zeros(3), np.zeros(3))
    assert m == {"max_abs": 0.0, "mean_rel": 0.0, "nonfinite": 0}
    m = oracle.error_metrics(np.zeros((0, 4)), np.zeros((0, 4)))
    assert m == {"max_abs": 0.0, "mean_rel": 0.0, "nonfinite": 0}


def test_lse_closed_form_on_the_two_key_example():
    """lse = log(exp(s0) + exp(s1) [+ exp(z)]) on the hand-derived two-key
    fixture; a single key gives lse = s0 exactly."""
    g = json.load(open(os.path.join(GOLDEN, "two_keys.json")))
    D = W.QK_DEPTH
    q, k0, k1 = np.zeros(D), np.zeros(D), np.zeros(D)
    for dst, src in ((q, g["q"]), (k0, g["k0"]), (k1, g["k1"])):
        for c, x in src.items():
            if int(c) < D:
                dst[int(c)] = x
    qt = torch.from_numpy(q).to(torch.bfloat16).reshape(1, 1, D).view(torch.int16).numpy().view(np.uint16)
    kv = torch.from_numpy(np.stack([k0, k1])).to(torch.float8_e4m3fn).view(torch.uint8).reshape(1, 2, D).numpy()
    # q = (1, 0.5), k0 = (1, 2, 3), k1 = (3, 0, -1): s0 = 2, s1 = 3 at scale 1
    s0, s1 = 2.0, 3.0
    for z, want in ((None, math.log(math.exp(s0) + math.exp(s1))),
                    (0.0, math.log(math.exp(s0) + math.exp(s1) + 1.0)),
                    (2.5, math.log(math.exp(s0) + math.exp(s1) + math.exp(2.5)))):
        res = oracle.sparse_mla_prefill(qt, kv, np.array([[0]], np.int32), np.array([0, 1], np.int32), None,
                                        np.array([[0, 1]], np.uint32), np.array([2], np.uint32),
                                        None if z is None else np.array([z], np.float32), 1.0, 0)
        assert abs(res["lse"][0, 0] - want) < 1e-12, z
    one = oracle.sparse_mla_prefill(qt, kv, np.array([[0]], np.int32), np.array([0, 1], np.int32), None,
                                    np.array([[0, 1]], np.uint32), np.array([1], np.uint32), None, 1.0, 0)
    assert one["lse"][0, 0] == s0
