"""The no-allocation entry point (sparse_mla_prefill_split_noalloc) against
the split entry point with a caller workspace, through the C ABI.

Both run the same kernels; only where the run partials live differs (the
library's fixed per-GPU scratch array instead of a workspace), so the outputs
must agree bit for bit.  Two calls in a row, the second smaller, check that
the scratch array's left-over contents from the first call do not leak into
the second.  The oracle is checked too, at the parity bar.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_token_amd as smla
import workloads as W

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    smla.load_library()


def make(T_per_seq, H, topk, sbs, sink, seed):
    s = W.CaseSpec(name="noalloc", num_seqs=2, q_per_seq=T_per_seq, ctx=topk + 80, q_pos0=topk + 70,
                   num_heads=H, topk=topk, page_size=64, shuffle_pages=True, lengths=f"uniform:1:{topk}",
                   scale_block_size=sbs, sink=sink)
    case = W.make_case(s, seed=seed, device="cpu")
    return case, case.host_arrays(), case.to("cuda")


def run_both(g, num_splits):
    T, H = g.q.shape[:2]
    ref_out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    smla.sparse_mla_prefill(g.q, g.kv_pages, g.page_table, g.cu_seqlens_q, g.indices, g.topk_lengths, g.scale,
                            g.scale_block_size, g.scales, g.sink, out=ref_out, num_splits=num_splits)
    out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    smla.sparse_mla_prefill_split_noalloc(g.q, g.kv_pages, g.page_table, g.cu_seqlens_q, g.indices, g.topk_lengths,
                                         g.scale, out, num_splits, g.scale_block_size, g.scales, g.sink)
    torch.cuda.synchronize()
    return out, ref_out


def check_against_oracle(out, a, label):
    ref = oracle.sparse_mla_prefill(a["q_bits"], a["kv_pages"], a["page_table"], a["cu_seqlens_q"], a["scales"],
                                    a["indices"], a["topk_lengths"], a["sink"], a["scale"],
                                    a["scale_block_size"])["out"]
    m = oracle.error_metrics(out.float().cpu().double().numpy(), ref)
    say(f"  {label}: max_abs={m['max_abs']:.3e} mean_rel={m['mean_rel']:.3e} nonfinite={m['nonfinite']}")
    assert m["nonfinite"] == 0 and m["max_abs"] <= 2e-2 and m["mean_rel"] <= 5e-3, (label, m)


@pytest.mark.parametrize("sbs,sink", [(0, False), (576, True), (32, True)])
def test_noalloc_matches_the_workspace_entry_twice(sbs, sink):
    say(f"case noalloc sbs={sbs} sink={sink}: call 1 (2 x 6 tokens, 128 heads, top-320, 3 runs)")
    _, a1, g1 = make(6, 128, 320, sbs, sink, seed=901 + sbs)
    out1, ref1 = run_both(g1, 3)
    assert torch.equal(out1, ref1)
    check_against_oracle(out1, a1, f"noalloc/sbs{sbs}/call1")
    say(f"case noalloc sbs={sbs} sink={sink}: call 2 (2 x 2 tokens, 64 heads, top-128, 2 runs)")
    _, a2, g2 = make(2, 64, 128, sbs, sink, seed=951 + sbs)
    out2, ref2 = run_both(g2, 2)
    assert torch.equal(out2, ref2)
    check_against_oracle(out2, a2, f"noalloc/sbs{sbs}/call2")


def test_noalloc_one_run_and_scratch_limit():
    say("case noalloc one run, then a request beyond the scratch array")
    _, a, g = make(3, 128, 192, 0, True, seed=977)
    out, ref = run_both(g, 1)
    assert torch.equal(out, ref)
    T, H = g.q.shape[:2]
    # 32 runs of 6 tokens x 128 heads fit; 4096 tokens in 3 runs do not, and
    # that error is returned on the host before anything is enqueued
    assert smla.split_workspace_bytes(T, H, 192, 32) <= smla.noalloc_scratch_bytes()
    big_T = 4096
    q = torch.zeros((big_T, H, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((big_T, 192), dtype=torch.int32, device="cuda")
    lens = torch.zeros((big_T,), dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, big_T], dtype=torch.int32, device="cuda")
    o = torch.empty((big_T, H, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(smla.SmlaError) as e:
        smla.sparse_mla_prefill_split_noalloc(q, g.kv_pages, g.page_table[:1].contiguous(), cu, idx, lens, g.scale,
                                             o, 3)
    assert e.value.status == 6
