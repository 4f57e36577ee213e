"""CPU float64 oracle for dense MLA prefill with a block-scaled FP8 K_rope.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes -- the "mla_sm100_prefill_blockscale" page (function
description, Parameters and Args) and the "SM100MLA" page (comptime members:
a 64-wide rope part of K): softmax attention of each query row over the keys
of its own sequence, where a key is the concatenation of a per-head K_nope
(BF16) and a K_rope shared by all heads and stored as FP8 with block scales,
which the kernel turns into BF16 before the matrix products:

    k_j = [k_nope[j, h_kv, 0:Dn] , decode_fp8(k_rope[j, 0:64]) * sigma(j, c)]
    s_j = scale * q[i, h, :] . k_j                     (q is [Dn + 64] wide)
    out[i, h, :] = sum_j softmax_j(s) v[j, h_kv, :]

Readings where the pages are silent (each listed with its reason in the
design notes):
  * sequences are padded to max_prompt_len rows in q and out (the page's
    output shape is [batch * num_rows, heads, depth]); with
    L_b = min(valid_length[b], max_prompt_len), row i of sequence b is valid
    when i < L_b and the keys of sequence b are its positions 0 .. L_b - 1 (a
    prefill of the whole prompt, so never more keys than rows); the page
    table holds at least max_prompt_len / P pages per sequence;
  * the mask is causal (key j visible to row i iff j <= i) or none (all
    valid keys); padding rows get zeros;
  * K_nope, V and K_rope live in paged caches that share one page table,
    row_j = page_table[b, j // P] * P + j % P, and a page id outside
    [0, num_pages) masks its keys (weight 0);
  * the K_rope block scale follows the sparse path's scale_block_size
    reading: 0 = unit scale, >= 64 = one f32 per row, smaller = one f32 per
    sbs-wide column block of the 64 rope columns (ceil(64 / sbs) per row,
    indexed by physical row);
  * group = heads / kv_heads query heads share a K_nope / V head
    (h_kv = h // group).
"""

from __future__ import annotations

import numpy as np

from .sparse_mla import decode_bf16, decode_e4m3fn

ROPE_DEPTH = 64


def rope_scale_columns(scale_block_size: int) -> int:
    """Columns of the K_rope scale table (0 for unit scale)."""
    if scale_block_size == 0:
        return 0
    if scale_block_size >= ROPE_DEPTH:
        return 1
    return -(-ROPE_DEPTH // scale_block_size)


def dense_rows(b: int, n_keys: int, page_table: np.ndarray, page_size: int, num_pages: int) -> np.ndarray:
    """Physical rows of keys 0 .. n_keys - 1 of sequence b; -1 where the page id
    is out of range."""
    j = np.arange(n_keys)
    pg = page_table[b, j // page_size].astype(np.int64)
    ok = (pg >= 0) & (pg < num_pages)
    return np.where(ok, pg * page_size + j % page_size, -1)


def dequant_rope(codes: np.ndarray, rows: np.ndarray, scales, scale_block_size: int) -> np.ndarray:
    """K_rope rows in float64: fp8 value times its block scale."""
    k = decode_e4m3fn(codes)                       # [n, 64]
    if scale_block_size == 0:
        return k
    sc = np.asarray(scales, dtype=np.float64)[rows]   # [n, ncols]
    if scale_block_size >= ROPE_DEPTH:
        return k * sc[:, :1]
    col_block = np.arange(ROPE_DEPTH) // scale_block_size
    return k * sc[:, col_block]


def mla_dense_prefill(q_bits, k_nope_bits, v_bits, k_rope_codes, k_rope_scales, page_table, valid_length,
                      scale: float, scale_block_size: int, max_prompt_len: int, causal: bool = True,
                      rows_subset=None):
    """Dense MLA prefill in float64.

    q_bits        u16 (bf16 bits) [B * S, H, Dn + 64]
    k_nope_bits   u16 [num_pages, P, Hkv, Dn]
    v_bits        u16 [num_pages, P, Hkv, Dv]
    k_rope_codes  u8  [num_pages, P, 64] (e4m3fn codes)
    k_rope_scales f32 [num_pages * P, ncols] or None (scale_block_size == 0)
    page_table    i32 [B, max_pages_per_seq]
    valid_length  u32 [B]
    rows_subset   optional list of global rows (b * S + i) to compute; the
                  others stay zero

    Returns a dict with out [B * S, H, Dv] and lse [B * S, H] (natural log,
    -inf for a row with no key).
    """
    q_bits = np.asarray(q_bits)
    BS, H, DQ = q_bits.shape
    num_pages, P, Hkv, Dn = k_nope_bits.shape
    Dv = v_bits.shape[3]
    assert DQ == Dn + ROPE_DEPTH and H % Hkv == 0
    group = H // Hkv
    S = max_prompt_len
    B = len(valid_length)
    assert BS == B * S
    kn_flat = k_nope_bits.reshape(num_pages * P, Hkv, Dn)
    v_flat = v_bits.reshape(num_pages * P, Hkv, Dv)
    kr_flat = k_rope_codes.reshape(num_pages * P, ROPE_DEPTH)
    out = np.zeros((BS, H, Dv))
    lse = np.full((BS, H), -np.inf)
    wanted = None if rows_subset is None else set(int(r) for r in rows_subset)
    for b in range(B):
        L = min(int(valid_length[b]), S)
        if L == 0:
            continue
        rows = dense_rows(b, L, page_table, P, num_pages)
        ok = rows >= 0
        r0 = np.where(ok, rows, 0)
        kr = dequant_rope(kr_flat[r0], r0, k_rope_scales, scale_block_size)      # [L, 64]
        for i in range(L):
            g = b * S + i
            if wanted is not None and g not in wanted:
                continue
            n = i + 1 if causal else L
            vis = ok[:n]
            if not vis.any():
                continue
            q = decode_bf16(q_bits[g])                                          # [H, DQ]
            for h in range(H):
                hk = h // group
                kn = decode_bf16(kn_flat[r0[:n], hk])                           # [n, Dn]
                s = scale * (kn @ q[h, :Dn] + kr[:n] @ q[h, Dn:])
                s = np.where(vis, s, -np.inf)
                m = s.max()
                w = np.exp(s - m)
                Z = w.sum()
                vv = decode_bf16(v_flat[r0[:n], hk])                            # [n, Dv]
                out[g, h] = (w / Z) @ np.where(vis[:, None], vv, 0.0)
                lse[g, h] = m + np.log(Z)
    return {"out": out, "lse": lse}


def dense_flops(valid_length, num_heads: int, qk_depth: int, v_depth: int, causal: bool = True) -> float:
    """Counted work: 2 * H * (Dqk + Dv) per visible (row, key) pair."""
    pairs = 0
    for L in valid_length:
        L = int(L)
        pairs += L * (L + 1) // 2 if causal else L * L
    return 2.0 * num_heads * (qk_depth + v_depth) * pairs
