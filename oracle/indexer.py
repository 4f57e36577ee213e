"""CPU float64 oracle for the FP8 lightning indexer and its top-k selection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes (the plain definitions, written out):

  Scores -- the "sparse_index_fp8_sm100" page (module description): for a
  query token t and a key j of the token's sequence,
      score[t, j] = k_scale[row_j] * sum_h relu(q[t, h, :] . k[row_j, :]) * q_scale[t, h]
  with q [tokens, heads, 128] and the paged keys [keys, 128] both FP8 e4m3,
  q_scale per (token, head) and k_scale per key.

  Top-k -- the pages feed these scores to a top-k stage they do not describe
  (same page: the kernel "is a drop-in for the score buffer the top-k stage
  consumes"); the plain reading taken here: the L = min(K, n_t) keys with the
  largest scores, ties going to the lower key index.

Readings where the pages are silent (listed with their reasons in the design
notes):
  * keys live in a paged cache like the attention's latent cache:
    row_j = page_table[b, j // P] * P + j % P, with k_scale indexed by that
    physical row; a page id outside [0, num_pages) masks the key (score -inf);
  * query tokens are packed by sequence (cu_seqlens_q) and are the last
    q_len_b positions of a sequence of seq_len_k[b] keys, so token i of the
    sequence sits at position pos = seq_len_k[b] - q_len_b + i and sees the
    causal key range [0, pos] (n_t = pos + 1 keys, none when pos < 0); the
    page leaves causal masking to a later slice, it is applied here in the
    score buffer: entries j >= n_t of a score row are -inf;
  * the selected keys are listed in ascending key order, the unused slots
    j >= L hold 0xFFFFFFFF, NaN scores order below -inf.
"""

from __future__ import annotations

import numpy as np

from .sparse_mla import decode_e4m3fn

INDEX_DEPTH = 128   # "sparse_index_fp8_sm100" page: MMA_K = depth = 128
UNUSED_SLOT = 0xFFFFFFFF


def causal_counts(cu_seqlens_q, seq_lens_k) -> np.ndarray:
    """n_t = number of keys query token t may see (its position + 1, >= 0)."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    lk = np.asarray(seq_lens_k, dtype=np.int64)
    n = np.zeros(int(cu[-1]), dtype=np.int64)
    for b in range(len(cu) - 1):
        q_len = cu[b + 1] - cu[b]
        for i in range(q_len):
            pos = lk[b] - q_len + i
            n[cu[b] + i] = max(pos + 1, 0)
    return n


def key_rows(b: int, n_keys: int, page_table, page_size: int, num_pages: int) -> np.ndarray:
    """Physical row of logical keys 0..n_keys-1 of sequence b (-1: page id out of range)."""
    j = np.arange(n_keys, dtype=np.int64)
    pt = np.asarray(page_table, dtype=np.int64)[b]
    logical_page = j // page_size
    pages = np.where(logical_page < pt.shape[0], pt[np.minimum(logical_page, pt.shape[0] - 1)], -1)
    ok = (pages >= 0) & (pages < num_pages) & (logical_page < pt.shape[0])
    return np.where(ok, pages * page_size + j % page_size, -1)


def indexer_scores(q_codes, q_scale, k_pages, k_scale, page_table, cu_seqlens_q, seq_lens_k,
                   score_stride: int, tokens=None) -> np.ndarray:
    """Score rows [n_tokens, score_stride] in float64 (-inf past the causal range).

    q_codes  uint8 [T, H, 128] e4m3fn codes;  q_scale float32 [T, H]
    k_pages  uint8 [num_pages, P, 128] e4m3fn codes;  k_scale float32 [num_pages * P]
    """
    q_codes = np.asarray(q_codes, dtype=np.uint8)
    T, H, D = q_codes.shape
    k_pages = np.asarray(k_pages, dtype=np.uint8)
    num_pages, P, _ = k_pages.shape
    flat_k = k_pages.reshape(-1, D)
    k_scale = np.asarray(k_scale, dtype=np.float64)
    q_scale = np.asarray(q_scale, dtype=np.float64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    n_t = causal_counts(cu_seqlens_q, seq_lens_k)
    if tokens is None:
        tokens = np.arange(T)
    out = np.full((len(tokens), score_stride), -np.inf)
    for i, t in enumerate(tokens):
        b = int(np.searchsorted(cu, t, side="right") - 1)
        n = int(min(n_t[t], score_stride))
        if n == 0:
            continue
        rows = key_rows(b, n, page_table, P, num_pages)
        ok = rows >= 0
        k = decode_e4m3fn(flat_k[np.where(ok, rows, 0)])        # [n, 128]
        q = decode_e4m3fn(q_codes[t])                            # [H, 128]
        dots = q @ k.T                                           # [H, n]
        s = (np.maximum(dots, 0.0) * q_scale[t][:, None]).sum(axis=0)
        s = s * k_scale[np.where(ok, rows, 0)]
        out[i, :n] = np.where(ok, s, -np.inf)
    return out


def topk_select(scores, n_valid, topk: int):
    """Top-k of each score row by (score descending, key index ascending).

    scores   [n, S] (any float type; compared as given)
    n_valid  [n] keys 0..n_valid-1 of each row take part
    Returns (indices uint32 [n, topk] ascending, UNUSED_SLOT-filled;
             lengths uint32 [n] = min(topk, n_valid)).
    """
    scores = np.asarray(scores)
    n_rows = scores.shape[0]
    idx = np.full((n_rows, topk), UNUSED_SLOT, dtype=np.uint32)
    lens = np.zeros(n_rows, dtype=np.uint32)
    for r in range(n_rows):
        n = int(min(n_valid[r], scores.shape[1]))
        L = min(topk, n)
        lens[r] = L
        if L == 0:
            continue
        s = scores[r, :n].astype(np.float64)
        key = np.where(np.isnan(s), -np.inf, s)
        nan_rank = np.isnan(s).astype(np.int64)      # NaN after -inf
        # np.lexsort sorts by the last array first: -key ascending (score
        # descending), then NaN after numbers, then index ascending
        order = np.lexsort((np.arange(n), nan_rank, -key))
        chosen = np.sort(order[:L])
        idx[r, :L] = chosen.astype(np.uint32)
    return idx, lens
