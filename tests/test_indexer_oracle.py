"""Pins of the indexer oracle (CPU): values fixed by hand arithmetic from the
score formula of the "sparse_index_fp8_sm100" page, invariants of that
formula, and the top-k reading checked against an exhaustive search."""

import itertools
import json
from pathlib import Path

import numpy as np
import pytest

import oracle

GOLDEN = Path(__file__).resolve().parent / "golden"

# e4m3fn codes: sign | exponent (bias 7) | 3 mantissa bits
E4M3 = {0.0: 0x00, 0.5: 0x30, 1.0: 0x38, 1.5: 0x3C, 2.0: 0x40, 3.0: 0x44, -1.0: 0xB8, -2.0: 0xC0}


def one_seq(q_codes, q_scale, k_rows, k_scale, seq_len_k=None, page_size=4):
    """Wrap single-sequence inputs: keys 0..n-1 in pages laid out in order."""
    n = k_rows.shape[0]
    pages = -(-n // page_size)
    kp = np.zeros((pages * page_size, oracle.INDEX_DEPTH), dtype=np.uint8)
    kp[:n] = k_rows
    ks = np.zeros(pages * page_size, dtype=np.float32)
    ks[:n] = k_scale
    T = q_codes.shape[0]
    return dict(q_codes=q_codes, q_scale=np.asarray(q_scale, dtype=np.float32),
                k_pages=kp.reshape(pages, page_size, -1), k_scale=ks,
                page_table=np.arange(pages, dtype=np.int32)[None, :],
                cu_seqlens_q=np.array([0, T], dtype=np.int32),
                seq_lens_k=np.array([n if seq_len_k is None else seq_len_k], dtype=np.int32))


def test_hand_computed_scores():
    # two heads; head 0: q = 1.0 at dim 5; head 1: q = 1.0 at dim 5 and 2.0 at dim 7
    q = np.zeros((1, 2, 128), dtype=np.uint8)
    q[0, 0, 5] = E4M3[1.0]
    q[0, 1, 5] = E4M3[1.0]
    q[0, 1, 7] = E4M3[2.0]
    # key 0: dim 5 = 3.0, dim 7 = -1.0 -> dots (3, 2*-1 + 3 = 1)
    # key 1: dim 5 = -1.0, dim 7 = 1.5 -> dots (-1, 2*1.5 - 1 = 2); relu drops head 0
    k = np.zeros((2, 128), dtype=np.uint8)
    k[0, 5], k[0, 7] = E4M3[3.0], E4M3[-1.0]
    k[1, 5], k[1, 7] = E4M3[-1.0], E4M3[1.5]
    a = one_seq(q, [[0.5, -2.0]], k, [4.0, 0.25])
    s = oracle.indexer_scores(**a, score_stride=4)
    # key 0: 4 * (3 * 0.5 + 1 * -2) = -2;  key 1: 0.25 * (0 + 2 * -2) = -1
    # the single query token sits at position 1 and sees keys 0 and 1
    assert s[0, 0] == -2.0 and s[0, 1] == -1.0
    assert np.isneginf(s[0, 2:]).all()


def test_relu_drops_negative_heads_and_scales_are_linear():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 0x7F, size=(1, 4, 128), dtype=np.uint8)   # positive codes only
    k = rng.integers(0, 0x7F, size=(6, 128), dtype=np.uint8)
    k[:, 0] = 0x00
    a = one_seq(q, np.ones((1, 4)), k, np.ones(6))
    base = oracle.indexer_scores(**a, score_stride=6)[0]
    assert (base > 0).all()                      # positive operands: relu is the identity
    # negating every key makes every dot product negative: all heads drop out
    kneg = k | 0x80
    a_neg = one_seq(q, np.ones((1, 4)), kneg, np.ones(6))
    assert (oracle.indexer_scores(**a_neg, score_stride=6)[0] == 0).all()
    # k_scale multiplies, q_scale weights heads linearly
    a2 = one_seq(q, np.full((1, 4), 3.0), k, np.full(6, 0.5))
    np.testing.assert_allclose(oracle.indexer_scores(**a2, score_stride=6)[0], 1.5 * base, rtol=1e-15)


def test_heads_add_up():
    rng = np.random.default_rng(4)
    q = rng.integers(0, 256, size=(2, 6, 128), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0          # no NaN codes
    k = rng.integers(0, 256, size=(9, 128), dtype=np.uint8)
    k[(k & 0x7F) == 0x7F] = 0
    qs = rng.normal(size=(2, 6)).astype(np.float32)
    ks = rng.uniform(0.5, 2, size=9).astype(np.float32)
    whole = oracle.indexer_scores(**one_seq(q, qs, k, ks), score_stride=9)
    part1 = oracle.indexer_scores(**one_seq(q[:, :2], qs[:, :2], k, ks), score_stride=9)
    part2 = oracle.indexer_scores(**one_seq(q[:, 2:], qs[:, 2:], k, ks), score_stride=9)
    fin = np.isfinite(whole)
    np.testing.assert_allclose(whole[fin], (part1 + part2)[fin], rtol=1e-12, atol=1e-9)
    assert (np.isfinite(part1) == fin).all()


def test_causal_counts_and_page_indirection():
    # two sequences: 3 queries over 5 keys (positions 2, 3, 4) and 2 queries over 2 keys (0, 1)
    n = oracle.causal_counts([0, 3, 5], [5, 2])
    assert n.tolist() == [3, 4, 5, 1, 2]
    # more queries than keys: leading queries see nothing
    assert oracle.causal_counts([0, 3], [1]).tolist() == [0, 0, 1]
    # shuffled physical pages give the same scores as an in-order layout
    rng = np.random.default_rng(5)
    P, pages = 4, 5
    q = rng.integers(0, 0x70, size=(3, 2, 128), dtype=np.uint8)
    k = rng.integers(0, 0x70, size=(pages * P, 128), dtype=np.uint8)
    ks = rng.uniform(0.5, 2, size=pages * P).astype(np.float32)
    qs = np.ones((3, 2), dtype=np.float32)
    a = one_seq(q, qs, k, ks, page_size=P)
    ref = oracle.indexer_scores(**a, score_stride=pages * P)
    perm = rng.permutation(pages)
    kp2 = np.zeros_like(a["k_pages"])
    ks2 = np.zeros_like(a["k_scale"])
    for logical, phys in enumerate(perm):
        kp2[phys] = a["k_pages"][logical]
        ks2[phys * P:(phys + 1) * P] = a["k_scale"][logical * P:(logical + 1) * P]
    a2 = dict(a, k_pages=kp2, k_scale=ks2, page_table=perm.astype(np.int32)[None, :])
    np.testing.assert_array_equal(oracle.indexer_scores(**a2, score_stride=pages * P), ref)
    # a page id out of range masks its keys
    bad = perm.copy()
    bad[1] = 99
    a3 = dict(a2, page_table=bad.astype(np.int32)[None, :])
    s3 = oracle.indexer_scores(**a3, score_stride=pages * P)
    assert np.isneginf(s3[:, P:2 * P]).all()
    np.testing.assert_array_equal(s3[:, :P], ref[:, :P])


def test_topk_golden_cases():
    cases = json.loads((GOLDEN / "topk_cases.json").read_text())["cases"]
    for c in cases:
        s = np.array([[np.nan if v == "nan" else float(v) for v in c["scores"]]], dtype=np.float32)
        idx, lens = oracle.topk_select(s, [c["n_valid"]], c["topk"])
        assert lens.tolist() == [c["length"]], c["name"]
        assert idx[0].tolist() == c["indices"] + [oracle.UNUSED_SLOT] * (c["topk"] - c["length"]), c["name"]


def brute_force_topk(s, L):
    """Best L-subset by exhaustive search: compare candidate subsets by their
    scores sorted descending, then by their indices (lower wins on ties)."""
    n = len(s)
    key = lambda v: (-np.inf if np.isnan(v) else v, 0 if not np.isnan(v) else -1)
    best = None
    for sub in itertools.combinations(range(n), L):
        vals = sorted(((key(s[i]), -i) for i in sub), reverse=True)
        if best is None or vals > best[0]:
            best = (vals, sub)
    return list(best[1])


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_exhaustive_search(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 10))
    # few distinct values: many ties
    s = rng.integers(-3, 3, size=n).astype(np.float32)
    if seed % 3 == 0:
        s[rng.integers(0, n)] = np.nan
    if seed % 4 == 1:
        s[rng.integers(0, n)] = -np.inf
    for L in range(0, n + 1):
        idx, lens = oracle.topk_select(s[None, :], [n], L)
        assert lens[0] == L
        assert idx[0, :L].tolist() == sorted(brute_force_topk(s, L)), (s, L)


def test_topk_invariants_on_a_long_row():
    rng = np.random.default_rng(7)
    n, K = 3000, 700
    s = np.round(rng.normal(size=n), 1).astype(np.float32)   # heavy ties
    idx, lens = oracle.topk_select(s[None, :], [n], K)
    sel = idx[0, :K].astype(np.int64)
    assert lens[0] == K and (np.diff(sel) > 0).all()
    rest = np.setdiff1d(np.arange(n), sel)
    assert s[sel].min() >= s[rest].max()
    thr = s[sel].min()
    # every key scoring exactly the threshold and left out has a larger index
    # than every such key taken
    assert sel[s[sel] == thr].max() < rest[s[rest] == thr].min()
