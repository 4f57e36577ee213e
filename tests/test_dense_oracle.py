"""Pins of the dense MLA prefill oracle (CPU): special cases that reduce to
PyTorch's scaled-dot-product attention, to the already pinned sparse oracle
(a dense causal prefill is the sparse attention over the key list 0 .. i),
closed forms, and hand-computed dequantisation values."""

import numpy as np
import pytest
import torch

import oracle
from oracle import dense_mla as D


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fp8_codes(x: torch.Tensor) -> np.ndarray:
    return x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make(B=2, S=24, H=4, Hkv=4, Dn=32, Dv=16, P=8, lens=(24, 17), seed=0, sbs=0, pages=None):
    g = torch.Generator().manual_seed(seed)
    maxp = -(-S // P)
    num_pages = pages if pages is not None else B * maxp
    q = bf16_bits(torch.randn(B * S, H, Dn + 64, generator=g))
    kn = bf16_bits(torch.randn(num_pages, P, Hkv, Dn, generator=g))
    v = bf16_bits(torch.randn(num_pages, P, Hkv, Dv, generator=g))
    kr = fp8_codes(torch.randn(num_pages, P, 64, generator=g) * 4)
    nc = D.rope_scale_columns(sbs)
    sc = None if nc == 0 else torch.exp2(torch.randint(-3, 3, (num_pages * P, nc), generator=g).float()).numpy()
    pt = np.arange(B * maxp, dtype=np.int32).reshape(B, maxp) % num_pages
    return dict(q_bits=q, k_nope_bits=kn, v_bits=v, k_rope_codes=kr, k_rope_scales=sc, page_table=pt,
                valid_length=np.array(lens, dtype=np.uint32), scale_block_size=sbs, max_prompt_len=S)


def sdpa_reference(a, scale, causal):
    """The same attention through torch's scaled_dot_product_attention (f64),
    one sequence at a time, keys laid out in order."""
    B = len(a["valid_length"])
    S = a["max_prompt_len"]
    num_pages, P, Hkv, Dn = a["k_nope_bits"].shape
    H = a["q_bits"].shape[1]
    out = np.zeros((B * S, H, a["v_bits"].shape[3]))
    for b in range(B):
        L = int(a["valid_length"][b])
        if L == 0:
            continue
        rows = a["page_table"][b, np.arange(L) // P].astype(np.int64) * P + np.arange(L) % P
        kn = oracle.decode_bf16(a["k_nope_bits"].reshape(-1, Hkv, Dn)[rows])          # [L, Hkv, Dn]
        kr = oracle.decode_e4m3fn(a["k_rope_codes"].reshape(-1, 64)[rows])              # [L, 64]
        if a["scale_block_size"]:
            sc = a["k_rope_scales"][rows]
            kr = kr * np.repeat(sc, 64 // sc.shape[1], axis=1)
        v = oracle.decode_bf16(a["v_bits"].reshape(-1, Hkv, a["v_bits"].shape[3])[rows])
        k = np.concatenate([kn, np.broadcast_to(kr[:, None, :], (L, Hkv, 64))], axis=2)
        q = oracle.decode_bf16(a["q_bits"][b * S:b * S + L])                            # [L, H, DQ]
        g = H // Hkv
        kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)
        vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
        qt = torch.from_numpy(q).permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
        out[b * S:b * S + L] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("sbs,Hkv", [(0, 4), (64, 2), (32, 1), (16, 4)])
def test_matches_scaled_dot_product_attention(causal, sbs, Hkv):
    a = make(sbs=sbs, Hkv=Hkv, seed=3 + sbs + Hkv)
    got = D.mla_dense_prefill(**a, scale=0.17, causal=causal)["out"]
    ref = sdpa_reference(a, 0.17, causal)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    # padding rows stay zero
    assert (got[24 + 17:48] == 0).all()


def test_is_the_sparse_attention_over_the_causal_key_list():
    # one K_nope / V head shared by all query heads, V = K_nope with values
    # exact in e4m3fn, scales per 32 columns: the sparse latent row
    # [k_nope | 0 ... | k_rope] with its first 128 columns as V gives the same
    # attention (columns 128 .. 511 of its output are 0)
    B, S, H, P = 1, 20, 3, 16
    g = torch.Generator().manual_seed(9)
    kn_f = torch.randn(2, P, 1, 128, generator=g).to(torch.float8_e4m3fn).float()
    kn = bf16_bits(kn_f)
    kr = fp8_codes(torch.randn(2, P, 64, generator=g) * 3)
    sc = torch.exp2(torch.randint(-2, 3, (2 * P, 2), generator=g).float()).numpy()
    q = bf16_bits(torch.randn(B * S, H, 192, generator=g))
    pt = np.array([[1, 0]], dtype=np.int32)
    dense = D.mla_dense_prefill(q, kn, kn, kr, sc, pt, np.array([S], np.uint32), 0.11, 32, S)["out"]

    latent = np.zeros((2, P, 576), dtype=np.uint8)
    latent[:, :, :128] = kn_f.to(torch.float8_e4m3fn).view(torch.uint8).numpy()[:, :, 0, :]
    latent[:, :, 512:] = kr
    scales18 = np.ones((2 * P, 18), dtype=np.float32)
    scales18[:, 16:] = sc
    qs = np.zeros((S, H, 576), dtype=np.uint16)
    qs[:, :, :128] = q[:, :, :128]
    qs[:, :, 512:] = q[:, :, 128:]
    idx = np.full((S, S), 0xFFFFFFFF, dtype=np.uint32)
    for i in range(S):
        idx[i, :i + 1] = np.arange(i + 1)
    sparse = oracle.sparse_mla_prefill(qs, latent, pt, np.array([0, S], np.int32), scales18, idx,
                                       np.arange(1, S + 1, dtype=np.uint32), None, 0.11, 32)["out"]
    np.testing.assert_allclose(dense, sparse[:, :, :128], rtol=1e-12, atol=1e-14)
    assert (sparse[:, :, 128:] == 0).all()


def test_closed_forms():
    a = make(B=1, S=12, H=2, Hkv=2, lens=(12,), seed=5)
    # q = 0: uniform weights, row i is the mean of v_0 .. v_i
    a0 = dict(a, q_bits=np.zeros_like(a["q_bits"]))
    out = D.mla_dense_prefill(**a0, scale=1.0)["out"]
    v = oracle.decode_bf16(a["v_bits"].reshape(-1, 2, 16))[:12]
    for i in range(12):
        np.testing.assert_allclose(out[i], v[:i + 1].mean(axis=0), rtol=1e-13, atol=1e-15)
    # row 0 sees one key: its value comes back exactly; lse = its logit
    r = D.mla_dense_prefill(**a, scale=0.3)
    assert np.array_equal(r["out"][0], v[0])
    # a length past max_prompt_len counts as max_prompt_len
    big = D.mla_dense_prefill(**dict(a, valid_length=np.array([1000], np.uint32)), scale=0.3, causal=False)
    np.testing.assert_array_equal(big["out"], D.mla_dense_prefill(**a, scale=0.3, causal=False)["out"])
    # a length-0 sequence produces zeros
    z = D.mla_dense_prefill(**dict(a, valid_length=np.array([0], np.uint32)), scale=0.3)
    assert (z["out"] == 0).all() and np.isneginf(z["lse"]).all()


def test_rope_dequantisation_by_hand():
    codes = np.zeros((2, 64), dtype=np.uint8)
    codes[0, 0], codes[0, 40] = 0x38, 0xC0       # 1.0, -2.0
    codes[1, 63] = 0x3C                          # 1.5
    sc = np.array([[0.5, 4.0], [2.0, 8.0]], dtype=np.float32)
    k = D.dequant_rope(codes, np.array([0, 1]), sc, 32)
    assert k[0, 0] == 0.5 and k[0, 40] == -8.0 and k[1, 63] == 12.0
    # one scale per row (column 0 of the table), taken from the physical row given
    k1 = D.dequant_rope(codes, np.array([1, 0]), sc, 64)
    assert k1[0, 0] == 2.0 and k1[0, 40] == -4.0 and k1[1, 63] == 0.75
    assert D.rope_scale_columns(0) == 0 and D.rope_scale_columns(64) == 1
    assert D.rope_scale_columns(576) == 1 and D.rope_scale_columns(48) == 2 and D.rope_scale_columns(16) == 4


def test_bad_pages_and_shuffled_pages():
    a = make(B=1, S=24, H=2, Hkv=2, P=8, lens=(24,), seed=6)
    ref = D.mla_dense_prefill(**a, scale=0.2, causal=False)["out"]
    # the same keys on shuffled physical pages
    perm = np.array([2, 0, 1])
    b = dict(a)
    for name in ("k_nope_bits", "v_bits", "k_rope_codes"):
        arr = np.zeros_like(a[name])
        arr[perm] = a[name]
        b[name] = arr
    b["page_table"] = perm[None, :].astype(np.int32)
    np.testing.assert_array_equal(D.mla_dense_prefill(**b, scale=0.2, causal=False)["out"], ref)
    # a bad page id drops its 8 keys: the same as SDPA over the other 16
    c = dict(a, page_table=np.array([[0, 99, 2]], dtype=np.int32))
    got = D.mla_dense_prefill(**c, scale=0.2, causal=False)["out"]
    keep = np.r_[0:8, 16:24]
    q = torch.from_numpy(oracle.decode_bf16(a["q_bits"][:24])).permute(1, 0, 2)
    kn = oracle.decode_bf16(a["k_nope_bits"].reshape(-1, 2, 32))[keep]
    kr = oracle.decode_e4m3fn(a["k_rope_codes"].reshape(-1, 64))[keep]
    k = torch.from_numpy(np.concatenate([kn, np.broadcast_to(kr[:, None], (16, 2, 64))], 2)).permute(1, 0, 2)
    v = torch.from_numpy(oracle.decode_bf16(a["v_bits"].reshape(-1, 2, 16))[keep]).permute(1, 0, 2)
    ref2 = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.2).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got[:24], ref2, rtol=1e-10, atol=1e-12)


def test_flop_count():
    assert D.dense_flops([4], 2, 192, 128) == 2 * 2 * 320 * 10
    assert D.dense_flops([4, 3], 1, 192, 128, causal=False) == 2 * 320 * 25
