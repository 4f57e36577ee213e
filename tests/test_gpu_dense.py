"""GPU parity of the dense MLA prefill (BF16 MFMA, block-scaled FP8 K_rope)
against the float64 oracle, through the C ABI.

Error budget: q, K_nope and V are BF16 and enter the products exactly; the
K_rope (fp8 x block scale) and P are rounded to BF16 (2^-9 relative each),
sums run in f32 and the output is rounded to BF16 (2^-9).  The bar is the one
of the sparse path: max |gpu - oracle| <= 2e-2 and
sum |gpu - oracle| / sum |oracle| <= 5e-3.  Exact: a row that sees a single
key returns that key's V row, padding rows are 0.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_token_amd as smla
import workloads as W

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_REL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    smla.load_library()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(g):
    s = g.spec
    out = smla.mla_dense_prefill(g.q, g.k_nope, g.v, g.k_rope, g.k_rope_scales, g.page_table, g.valid_length,
                                 g.scale, s.scale_block_size, s.max_prompt_len, s.causal)
    torch.cuda.synchronize()
    return out


def check(out, ref, label):
    got = out.float().cpu().double().numpy()
    m = oracle.error_metrics(got, ref)
    say(f"  {label}: max_abs={m['max_abs']:.3e} mean_rel={m['mean_rel']:.3e} nonfinite={m['nonfinite']}")
    assert m["nonfinite"] == 0, label
    assert m["max_abs"] <= MAX_ABS, (label, m)
    assert m["mean_rel"] <= MEAN_REL, (label, m)


def case(spec, seed):
    c = W.make_dense_case(spec, seed, device="cpu")
    return c, c.host_arrays(), c.to("cuda")


def test_tiny():
    spec = W.DENSE_CONFIGS["dense_tiny"]
    say(f"case {spec}")
    c, a, g = case(spec, W.DENSE_SEEDS["dense_tiny"])
    check(run(g), oracle.mla_dense_prefill(**a)["out"], "dense_tiny")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("sbs", [0, 16, 32, 48, 64])
def test_scale_modes_and_masks(sbs, causal):
    spec = W.DenseSpec("modes", num_seqs=2, max_prompt_len=300, lengths=(300, 77), num_heads=8, page_size=64,
                       scale_block_size=sbs, causal=causal)
    say(f"case sbs={sbs} causal={causal}")
    c, a, g = case(spec, 3100 + sbs + int(causal))
    check(run(g), oracle.mla_dense_prefill(**a)["out"], f"sbs{sbs}/causal{int(causal)}")


@pytest.mark.parametrize("H,Hkv", [(8, 8), (8, 2), (6, 1), (3, 3)])
@pytest.mark.parametrize("P", [1, 16, 48, 96, 128])
def test_heads_groups_and_page_sizes(H, Hkv, P):
    spec = W.DenseSpec("groups", num_seqs=3, max_prompt_len=150, lengths=(150, 129, 64), num_heads=H,
                       num_kv_heads=Hkv, page_size=P, spare_pages=3)
    say(f"case H={H} Hkv={Hkv} P={P}")
    c, a, g = case(spec, 3200 + 7 * H + Hkv + P)
    check(run(g), oracle.mla_dense_prefill(**a)["out"], f"H{H}/Hkv{Hkv}/P{P}")


def test_ragged_lengths_bad_pages_and_padding():
    # lengths 0, 1, 65, 257 and one past S (counts as S); one page id out of range
    spec = W.DenseSpec("ragged", num_seqs=5, max_prompt_len=260, lengths=(0, 1, 65, 257, 1000), num_heads=4,
                       page_size=32)
    say("case ragged")
    c, a, g = case(spec, 3301)
    a["page_table"] = a["page_table"].copy()
    a["page_table"][4, 2] = 10 ** 6
    g.page_table.copy_(torch.from_numpy(a["page_table"]))
    out = run(g)
    ref = oracle.mla_dense_prefill(**a)["out"]
    check(out, ref, "ragged")
    got = out.float().cpu().numpy()
    S = spec.max_prompt_len
    assert (got[0:S] == 0).all()                       # an empty sequence
    assert (got[S + 1:2 * S] == 0).all()               # padding rows of the length-1 sequence
    assert (got[3 * S + 257:4 * S] == 0).all()


@pytest.mark.parametrize("H", [4, 128])
def test_one_visible_key_returns_the_row_exactly(H):
    # causal row 0 sees key 0 only: p = 1 and the output is V[key 0], exact in bf16
    spec = W.DenseSpec("first", num_seqs=2, max_prompt_len=130, lengths=(130, 5), num_heads=H, page_size=16)
    say(f"case first row H={H}")
    c, a, g = case(spec, 3401 + H)
    out = run(g)
    S = spec.max_prompt_len
    for b in range(2):
        ref = oracle.mla_dense_prefill(**a, rows_subset=[b * S])["out"][b * S]
        assert np.array_equal(out[b * S].float().cpu().double().numpy(), ref)


def test_repeat_calls_are_bit_identical():
    spec = W.DenseSpec("det", num_seqs=2, max_prompt_len=300, lengths=(300, 211), num_heads=8)
    c, a, g = case(spec, 3501)
    o1 = run(g).clone()
    assert torch.equal(o1, run(g))


def test_dense_dsv3_full_size_sampled():
    spec = W.DENSE_CONFIGS["dense_dsv3"]
    say(f"case {spec.name} full size, sampled rows")
    g = W.make_dense_case(spec, W.DENSE_SEEDS["dense_dsv3"], device="cuda")
    out = run(g)
    S = spec.max_prompt_len
    rows = [0, 127, 128, 2049, S - 1, S + 63, S + 3000, 2 * S - 1]
    a = g.to("cpu").host_arrays()
    ref = oracle.mla_dense_prefill(**a, rows_subset=rows)["out"]
    check(out[rows], ref[rows], "dense_dsv3 sampled")
