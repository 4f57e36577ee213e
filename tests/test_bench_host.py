"""Host-side checks of bench.py: the algorithmic byte count behind the HBM
roof, the kernel each scale mode and head count is reported against, the
source-hash guard on stored counter traffic, and the one-GPU exit.  CPU only."""

import json
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_algorithmic_bytes_counts_the_pool_once_when_it_fits_the_cache():
    spec = W.CONFIGS["tiny"]
    case = W.make_case(spec, seed=W.SEEDS["tiny"])
    T, H, K = spec.num_tokens, spec.num_heads, spec.topk
    keys = int(case.topk_lengths.clamp(max=K).sum())
    total, gathered = bench.algorithmic_bytes(case)
    fixed = T * H * 576 * 2 + T * H * 512 * 2 + T * K * 4 + T * 4
    assert gathered == keys * 576
    assert total == fixed + spec.num_pages * spec.page_size * 576


def test_algorithmic_bytes_counts_every_gathered_row_when_the_pool_does_not_fit(monkeypatch):
    spec = W.scaled(W.CONFIGS["tiny"], scale_block_size=32)
    case = W.make_case(spec, seed=5)
    monkeypatch.setattr(bench, "CACHE_BYTES", 0)
    total, gathered = bench.algorithmic_bytes(case)
    keys = int(case.topk_lengths.clamp(max=spec.topk).sum())
    ncols = case.scales.shape[1]
    assert ncols == 18
    assert gathered == keys * (576 + 4 * ncols)
    T, H, K = spec.num_tokens, spec.num_heads, spec.topk
    assert total == T * H * 576 * 2 + T * H * 512 * 2 + T * K * 4 + T * 4 + gathered


@pytest.mark.parametrize("H,sbs,kernel,issued", [
    (128, 0, "smla_fp8x2_kernel", 2.0),
    (128, 576, "smla_fp8x2_kernel", 2.0),
    (64, 0, "smla_fp8pair_kernel", 2.0),
    (16, 4096, "smla_fp8pair_kernel", 2.0),
    (128, 32, "smla_f16_wide_kernel", 1.0),
    (96, 32, "smla_f16_wide_kernel", 1.0),
    (64, 32, "smla_f16_block_kernel", 1.0),
])
def test_kernel_reported_for_each_mode(H, sbs, kernel, issued):
    spec = W.scaled(W.CONFIGS["tiny"], num_heads=H, scale_block_size=sbs)
    name, _, peak, per = bench.kernel_of(spec)
    assert name == kernel and per == issued
    assert peak == (bench.PEAK_FP16_TFLOPS if sbs and sbs < 576 else bench.PEAK_FP8_TFLOPS)
    name1, _, _, per1 = bench.kernel_of(spec, single_pass=True)
    if sbs == 0 or sbs >= 576:
        assert per1 == 1.0 and name1.endswith("(single pass)")


def test_decode_sized_batches_take_the_paired_kernel_in_one_run():
    # 128 tokens x two 64-head groups fill the 256 CUs: one run, paired kernel
    import sparse_mla_attention_token_amd as smla
    spec = W.CONFIGS["decode"]
    assert spec.num_tokens * 2 >= 256 > spec.num_tokens and spec.num_heads == 128
    assert bench.kernel_of(spec)[0] == "smla_fp8pair_kernel"
    assert smla.auto_splits(spec.num_tokens, spec.num_heads, spec.topk, 0) == 1
    # fewer tokens: split runs of the one-workgroup kernel
    small = W.scaled(spec, num_seqs=32)
    assert small.num_tokens * 2 < 256
    assert bench.kernel_of(small)[0] == "smla_fp8x2_kernel"
    assert smla.auto_splits(small.num_tokens, small.num_heads, small.topk, 0) > 1
    # a whole chip of tokens: one workgroup per token
    assert bench.kernel_of(W.CONFIGS["dsv32"])[0] == "smla_fp8x2_kernel"


def test_stored_traffic_is_dropped_once_the_sources_change(tmp_path, monkeypatch):
    rec = {"source_hash": bench.source_hash(), "bytes_per_launch": 123.0}
    f = tmp_path / "traffic_x.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "traffic_file", lambda w: f)
    assert bench.measured_traffic("x", "two-pass") == 123.0
    assert bench.measured_traffic("x", "single-pass") is None
    rec["source_hash"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic("x", "two-pass") is None


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout
