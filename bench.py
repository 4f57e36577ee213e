#!/usr/bin/env python3
"""Sparse MLA prefill benchmark (one GPU).

One step = one call of the attention over the whole DeepSeek-V3.2-shaped
workload (4096 query tokens x 128 heads x top-2048 listed keys of a paged FP8
latent cache, unit scale).  Prints one JSON line with TFLOP/s (2 * H * 1088
FLOP per gathered key), ms per call, the roofline of the attention kernel and
the CPU float64 oracle timed on a bounded token sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "sparse-MLA TFLOP/s + ms/call, 4096 tok × 128 heads × top-2048 FP8 KV"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, published
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense FP16 / BF16 MFMA, published
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E, published
CACHE_BYTES = 256 << 20      # MI355X Infinity Cache: a larger latent pool is gathered from HBM


def kernel_of(spec, single_pass=False):
    """(kernel, MFMA dtype, dense peak TFLOP/s, issued / counted FLOP) of the path
    the library dispatches for this scale mode."""
    sbs = spec.scale_block_size
    if sbs == 0 or sbs >= 576:
        # up to 64 heads, or fewer tokens than CUs whose 64-head groups fill
        # them (one run): the paired-wave kernel; else one workgroup per token
        T, H = spec.num_tokens, spec.num_heads
        heads_fill = H > 64 and T < 256 and T * ((H + 63) // 64) >= 256
        k = "smla_fp8pair_kernel" if H <= 64 or heads_fill else "smla_fp8x2_kernel"
        if single_pass:
            return k + " (single pass)", "fp8", PEAK_FP8_TFLOPS, 1.0
        # q and P each as two FP8 terms: every counted FLOP is issued twice
        return k, "fp8", PEAK_FP8_TFLOPS, 2.0
    # blockwise: one workgroup per token; 32 heads per wave above 64 heads
    k = "smla_f16_wide_kernel" if spec.num_heads > 64 else "smla_f16_block_kernel"
    return k, "fp16", PEAK_FP16_TFLOPS, 1.0


def algorithmic_bytes(case):
    """HBM bytes one attention launch must move: q, out, the index lists and
    lengths, and the latent pool -- each gathered row (576 bytes plus its
    scales) when the pool does not fit the cache, else the pool once."""
    import torch

    spec = case.spec
    T, H = spec.num_tokens, spec.num_heads
    ncols = 0 if case.scales is None else case.scales.shape[1]
    row_bytes = 576 + 4 * ncols
    keys = torch.clamp(case.topk_lengths.to(torch.int64), max=spec.topk).sum().item()
    pool = case.kv_pages.numel() + (0 if case.scales is None else case.scales.numel() * 4)
    fixed = T * H * 576 * 2 + T * H * 512 * 2 + case.indices.numel() * 4 + T * 4
    gathered = keys * row_bytes
    return fixed + (gathered if pool > CACHE_BYTES else pool), gathered


def traffic_file(workload):
    return ROOT / "profiles" / f"traffic_{workload}.json"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted((ROOT / "sparse_mla_attention_token_amd" / "csrc").glob("*")):
        h.update(p.name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(workload, variant):
    """HBM bytes per launch from committed rocprofv3 counter runs, only while
    the kernel sources are the ones the counters were taken on."""
    f = traffic_file(workload)
    if not f.exists():
        return None
    rec = json.loads(f.read_text())
    if rec.get("source_hash") != source_hash() or rec.get("variant", "two-pass") != variant:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(case, out_gpu, budget_s, max_tokens):
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    import workloads as W

    T = case.spec.num_tokens
    rng = np.random.default_rng(2024)
    order = rng.permutation(T)
    done, elapsed, refs = [], 0.0, []
    batch = 4
    cache = {}
    while elapsed < budget_s and len(done) < max_tokens and len(done) < T:
        toks = np.sort(order[len(done):len(done) + batch])
        a = W.subset_host_arrays(case, toks, cache)
        t0 = time.perf_counter()
        r = oracle.sparse_mla_prefill(a["q_bits"], a["kv_pages"], a["page_table"], a["cu_seqlens_q"],
                                      a["scales"], a["indices"], a["topk_lengths"], a["sink"], a["scale"],
                                      a["scale_block_size"])
        elapsed += time.perf_counter() - t0
        done.extend(toks.tolist())
        refs.append(r["out"])
    toks = np.array(done)
    flops = W.flops_of(case, toks)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    got = out_gpu[torch.from_numpy(toks).to(out_gpu.device)].float().cpu().double().numpy()
    m = oracle.error_metrics(got, np.concatenate(refs, axis=0))
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(toks)} of {T} query tokens (all heads, all listed keys), {elapsed:.1f} s; "
                  f"numpy float64, BLAS threads={threads}, os.cpu_count()={os.cpu_count()}",
        "seconds": elapsed,
        "tokens": int(len(toks)),
        "parity_vs_gpu": {"max_abs": m["max_abs"], "mean_rel": m["mean_rel"], "nonfinite": m["nonfinite"]},
    }


def indexer_main(args):
    """The FP8 lightning indexer (scores + top-k) on an indexer workload."""
    import numpy as np
    import torch

    import sparse_mla_attention_token_amd as smla
    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    smla.load_library()
    spec = W.INDEXER_CONFIGS[args.workload]
    log(f"generating workload {spec}")
    case = W.make_indexer_case(spec, W.INDEXER_SEEDS[args.workload], device="cuda")
    flops = W.indexer_flops(case)
    stream = torch.cuda.current_stream()
    copy_calibration(args.copy_mib)
    scores = torch.empty((spec.num_tokens, spec.stride), dtype=torch.float32, device="cuda")
    idx = torch.empty((spec.num_tokens, spec.topk), dtype=torch.int32, device="cuda")
    lens = torch.empty((spec.num_tokens,), dtype=torch.int32, device="cuda")

    def run_scores():
        smla.sparse_mla_index_scores(case.q, case.q_scale, case.k_pages, case.k_scale, case.page_table,
                                     case.cu_seqlens_q, case.seq_lens_k, spec.stride, scores=scores, stream=stream)

    def run_topk():
        smla.sparse_mla_index_topk(scores, case.cu_seqlens_q, case.seq_lens_k, spec.topk, indices=idx,
                                   topk_lengths=lens, stream=stream)

    def timed(fn, steps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    settle_clocks(lambda: (run_scores(), run_topk()), stream, args.settle_ms)
    ms_scores = timed(run_scores, args.steps)
    ms_topk = timed(run_topk, args.steps)
    ms = ms_scores + ms_topk
    tflops = flops / (ms * 1e-3) / 1e12
    score_tflops = flops / (ms_scores * 1e-3) / 1e12
    log(f"{args.workload}: scores {ms_scores:.4f} ms ({score_tflops:.1f} TFLOP/s), top-k {ms_topk:.4f} ms")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        a = case.to("cpu").host_arrays()
        rng = np.random.default_rng(2024)
        order = rng.permutation(spec.num_tokens)
        done, elapsed = [], 0.0
        while elapsed < args.cpu_seconds and len(done) < spec.num_tokens:
            toks = np.sort(order[len(done):len(done) + 8])
            t0 = time.perf_counter()
            oracle.indexer_scores(**a, score_stride=spec.stride, tokens=toks)
            elapsed += time.perf_counter() - t0
            done.extend(toks.tolist())
        n_t = oracle.causal_counts(a["cu_seqlens_q"], a["seq_lens_k"])
        sample_flops = 2.0 * spec.num_heads * W.INDEX_DEPTH * float(np.minimum(n_t[done], spec.stride).sum())
        cpu = {"value": sample_flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": os.cpu_count(),
               "kind": "oracle",
               "sample": f"scores of {len(done)} of {spec.num_tokens} query tokens (all heads, every visible key), "
                         f"{elapsed:.1f} s; numpy float64"}
    line = {
        "metric": "FP8 lightning-indexer TFLOP/s (scores + top-k), 2*H*128 FLOP per visible (token, key)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {spec.num_seqs} seq x {spec.q_per_seq} query tokens over "
                               f"{spec.ctx} keys, {spec.num_heads} heads, depth 128, top-{spec.topk}, page "
                               f"{spec.page_size}", "ms_scores": ms_scores, "ms_topk": ms_topk,
                   "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": score_tflops, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": score_tflops / PEAK_FP8_TFLOPS, "traffic": measured_traffic(args.workload, "two-pass"),
                     "kernel": "smla_index_score_kernel"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def copy_calibration(mibs):
    """Plain copy kernels of known sizes (a comma-separated list of MiB): their
    FETCH_SIZE / WRITE_SIZE counters calibrate a kernel's HBM traffic in
    profiler runs."""
    import torch
    for mib in [int(x) for x in str(mibs).split(",") if x.strip() and int(x) > 0]:
        src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {mib} MiB read + {mib} MiB written")
        del src, dst


def settle_clocks(fn, stream, settle_ms):
    """Run fn back to back on `stream` until settle_ms of GPU time have
    passed (outside any timed region).  The GPU leaves its idle clocks only
    after tens of milliseconds of sustained load, longer than the warm-up
    calls of a workload of a few milliseconds or less take; the timed calls
    then run at the clocks a busy GPU holds.  Returns (calls, ms)."""
    import torch

    if settle_ms <= 0:
        return 0, 0.0
    calls, spent, batch = 0, 0.0, 1
    while spent < settle_ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        spent += e0.elapsed_time(e1)
        calls += batch
        batch = min(batch * 2, 256)
    return calls, spent


def dense_main(args):
    """Dense MLA prefill with a block-scaled FP8 K_rope on a dense workload."""
    import numpy as np
    import torch

    import sparse_mla_attention_token_amd as smla
    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    smla.load_library()
    spec = W.DENSE_CONFIGS[args.workload]
    log(f"generating workload {spec}")
    case = W.make_dense_case(spec, W.DENSE_SEEDS[args.workload], device="cuda")
    flops = W.dense_flops(spec)
    stream = torch.cuda.current_stream()
    out = torch.empty((spec.num_seqs * spec.max_prompt_len, spec.num_heads, 128), dtype=torch.bfloat16,
                      device="cuda")

    copy_calibration(args.copy_mib)

    def step():
        smla.mla_dense_prefill(case.q, case.k_nope, case.v, case.k_rope, case.k_rope_scales, case.page_table,
                               case.valid_length, case.scale, spec.scale_block_size, spec.max_prompt_len,
                               spec.causal, out=out, stream=stream)

    settle_calls, settle_ms = settle_clocks(step, stream, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{args.workload}: {ms:.4f} ms, {tflops:.1f} TFLOP/s")

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        a = case.to("cpu").host_arrays()
        S = spec.max_prompt_len
        lens = [min(int(x), S) for x in spec.valid_lengths]
        valid = np.array([b * S + i for b in range(spec.num_seqs) for i in range(lens[b])])
        rng = np.random.default_rng(2025)
        order = rng.permutation(valid)
        done, elapsed, pairs = [], 0.0, 0
        while elapsed < args.cpu_seconds and len(done) < len(order):
            r = int(order[len(done)])
            t0 = time.perf_counter()
            oracle.mla_dense_prefill(**a, rows_subset=[r])
            elapsed += time.perf_counter() - t0
            done.append(r)
            pairs += (r % S) + 1 if spec.causal else lens[r // S]
        cpu = {"value": 2.0 * spec.num_heads * 320 * pairs / elapsed / 1e12, "unit": "TFLOP/s",
               "cores": os.cpu_count(), "kind": "oracle",
               "sample": f"{len(done)} random query rows (all heads, every visible key), {elapsed:.1f} s; "
                         f"numpy float64"}
    line = {
        "metric": "dense MLA prefill TFLOP/s (block-scaled FP8 K_rope), 2*H*(192+128) FLOP per visible (row, key)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {spec.num_seqs} seq x {spec.max_prompt_len} rows, lengths "
                               f"{list(spec.valid_lengths)}, {spec.num_heads} heads ({spec.kv_heads} kv), q 192 = "
                               f"128 nope + 64 rope, v 128, causal {spec.causal}, K_rope scale_block_size "
                               f"{spec.scale_block_size}, page {spec.page_size}", "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_FP16_TFLOPS, "traffic": measured_traffic(args.workload, "two-pass"),
                     "kernel": "smla_dense_kernel"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def probe_main(args):
    """Measured ceilings: back-to-back MFMA loops (peak_fp8 / peak_fp16 /
    peak_bf16, and peak_fp16_16x16 / peak_bf16_16x16 for the 16x16x32 shapes)
    and the attention's row gather alone (gather_hbm: random rows
    of a 1 GiB pool, beyond the 256 MB Infinity Cache; gather_l2: random rows of
    a 4.7 MB pool, the DSv3.2 prefill's, resident in L2), and coexec: how much
    independent VALU work a SIMD overlaps with FP8 MFMAs, from one wave or
    from a second wave on the same SIMD."""
    import torch

    from sparse_mla_attention_token_amd import probe

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        settle_clocks(fn, stream, args.settle_ms)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    w = args.workload
    if w == "coexec":
        # cycles per MFMA (and per VALU iteration) of the issue-behaviour probe,
        # one workgroup per CU, median over the CUs
        blocks, iters = 256, 4000
        cycles = torch.zeros(8 * blocks, dtype=torch.int64, device="cuda")
        out = torch.empty(8 * blocks, dtype=torch.float32, device="cuda")
        table = {}
        for mode, name in ((0, "one wave per SIMD, one dependent MFMA chain, N FMAs after each MFMA"),
                           (1, "one wave per SIMD, two independent MFMA chains alternating, N FMAs after each MFMA"),
                           (2, "two waves per SIMD: an MFMA-chain wave and a wave of N FMAs per iteration")):
            rows = {}
            for n in (0, 4, 8, 16):
                probe.coexec(mode, n, iters, blocks, cycles, out, stream)
                torch.cuda.synchronize()
                c = cycles.view(blocks, 8).double().median(dim=0).values.cpu()
                per = float(c[0]) / iters / (2 if mode == 1 else 1)
                rows[f"N={n}"] = ({"mfma_wave_cycles_per_mfma": round(per, 1),
                                   "valu_wave_cycles_per_iteration": round(float(c[4]) / iters, 1)}
                                  if mode == 2 else {"cycles_per_mfma": round(per, 1)})
            table[name] = rows
        line = {"metric": "issue behaviour of a SIMD: FP8 32x32x64 MFMA with independent v_fma_f32 work "
                          "(cycles per MFMA; 64 = the matrix pipe alone)",
                "value": table["two waves per SIMD: an MFMA-chain wave and a wave of N FMAs per iteration"]["N=16"][
                    "mfma_wave_cycles_per_mfma"],
                "unit": "cycles per MFMA", "n_gpus": 1, "higher_is_better": False,
                "config": {"workload": f"coexec: {blocks} workgroups x 8 waves x {iters} iterations"},
                "table": table}
        print(json.dumps(line), flush=True)
        return
    if w.startswith("peak_"):
        kind = w[len("peak_"):]
        blocks, iters = 1024, 8000
        out = torch.empty(4 * blocks, dtype=torch.float32, device="cuda")
        flop = probe.mfma(kind, iters, blocks, out, stream)
        ms = timed(lambda: probe.mfma(kind, iters, blocks, out, stream), args.steps)
        peak = PEAK_FP8_TFLOPS if kind == "fp8" else PEAK_FP16_TFLOPS
        value = flop / (ms * 1e-3) / 1e12
        shape = {"fp8": "v_mfma_scale_f32_32x32x64_f8f6f4", "fp16": "v_mfma_f32_32x32x16_f16",
                 "bf16": "v_mfma_f32_32x32x16_bf16", "fp16_16x16": "v_mfma_f32_16x16x32_f16",
                 "bf16_16x16": "v_mfma_f32_16x16x32_bf16"}[kind]
        line = {"metric": f"measured dense {kind} MFMA rate ({shape}, back to back, four accumulators per wave)",
                "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": ms, "higher_is_better": True, "published_peak": peak, "frac_of_published": value / peak,
                "config": {"workload": f"{w}: {blocks} workgroups x 4 waves x {iters} steps x 4 MFMAs",
                           "flop_per_step": flop}}
    else:
        big = w == "gather_hbm"
        pool_bytes = (1 << 30) if big else 8192 * 576
        nrows = pool_bytes // 576
        blocks, tiles = 1024, 32
        pool = torch.zeros(pool_bytes, dtype=torch.uint8, device="cuda")
        g = torch.Generator(device="cpu").manual_seed(77)
        rows = torch.randint(0, nrows, (blocks * tiles * 64,), generator=g, dtype=torch.int64).to(
            torch.int32).to("cuda")
        out = torch.empty(blocks, dtype=torch.int32, device="cuda")
        ms = timed(lambda: probe.gather(pool, rows, tiles, blocks, out, stream), args.steps)
        nbytes = blocks * tiles * 64 * 576
        value = nbytes / (ms * 1e-3) / 1e9
        line = {"metric": "measured rate of the attention's row gather alone (64 random 576-byte rows per tile, "
                          "global->LDS copies, two-stage ring)",
                "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": ms, "higher_is_better": True,
                "published_peak": PEAK_HBM_GBPS if big else None,
                "frac_of_published": value / PEAK_HBM_GBPS if big else None,
                "config": {"workload": f"{w}: {blocks} workgroups x {tiles} tiles of 64 rows from a "
                                       f"{pool_bytes / 1e6:.1f} MB pool", "bytes_per_step": nbytes}}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv32")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time budget (0 disables)")
    ap.add_argument("--cpu-max-tokens", type=int, default=1024)
    ap.add_argument("--variant", choices=("two-pass", "single-pass"), default="two-pass",
                    help="single-pass: q and P as one FP8 operand each (faster, percent-level error, "
                         "reported in cpu_baseline.parity_vs_gpu); never the default")
    ap.add_argument("--cold-calls", type=int, default=5,
                    help="calls timed one by one after a 512 MiB flush write (0 disables)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="before the cold calls and the warm-up, run the workload back to back for this "
                         "much GPU time so that the clocks leave their idle state (0 disables)")
    ap.add_argument("--copy-mib", default="0",
                    help="also run plain device copies of these many MiB, comma-separated (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the attention is timed on a single MI355X; sharding "
                                   "across GPUs is a design note, not built",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    if args.workload.startswith("peak_") or args.workload.startswith("gather_") or args.workload == "coexec":
        return probe_main(args)
    if args.workload.startswith("indexer"):
        return indexer_main(args)
    if args.workload.startswith("dense"):
        return dense_main(args)

    import torch

    import sparse_mla_attention_token_amd as smla
    import workloads as W

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    smla.load_library()
    spec = W.CONFIGS[args.workload]
    seed = W.SEEDS[args.workload]
    log(f"generating workload {spec}")
    case = W.make_case(spec, seed=seed, device="cuda")
    flops = W.flops_of(case)
    stream = torch.cuda.current_stream()
    out = torch.empty((spec.num_tokens, spec.num_heads, W.V_DEPTH), dtype=torch.bfloat16, device="cuda")

    # the library's run count (1 unless the tokens leave CUs idle); the split
    # workspace is allocated once, outside the timed region
    splits = smla.auto_splits(spec.num_tokens, spec.num_heads, spec.topk, spec.scale_block_size)
    ws = None
    if splits > 1:
        ws = torch.empty(smla.split_workspace_bytes(spec.num_tokens, spec.num_heads, spec.topk, splits),
                         dtype=torch.uint8, device="cuda")

    single = args.variant == "single-pass"

    def step():
        smla.sparse_mla_prefill(case.q, case.kv_pages, case.page_table, case.cu_seqlens_q, case.indices,
                                case.topk_lengths, case.scale, case.scale_block_size, case.scales, case.sink,
                                out=out, stream=stream, num_splits=splits, workspace=ws, single_pass=single)

    copy_calibration(args.copy_mib)

    settle_calls, settle_ms = settle_clocks(step, stream, args.settle_ms)

    # cold calls, before the warm-up and outside the timed region: a 512 MiB
    # write on the launch stream evicts the latent pool, q and the index lists
    # from L2 and the Infinity Cache before each call, which is timed alone
    cold_ms = None
    if args.cold_calls > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(args.cold_calls):
            flush.fill_(1)
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        cold_ms = sorted(times)[len(times) // 2]
        del flush
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps  # one attention launch per step (+ the combine when splits > 1)
    tflops = flops / (ms * 1e-3) / 1e12

    kname, kdtype, peak, issued = kernel_of(spec, single)
    hbm_bytes, gathered = algorithmic_bytes(case)
    hbm_gbps = hbm_bytes / (ms * 1e-3) / 1e9
    log(f"{args.workload}: {ms:.4f} ms/call, {tflops:.1f} TFLOP/s, {hbm_gbps:.0f} GB/s algorithmic HBM, "
        f"gather {gathered / (ms * 1e-3) / 1e9:.0f} GB/s")

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(case, out, args.cpu_seconds, args.cpu_max_tokens)
        log(f"cpu baseline: {cpu['value']:.5f} TFLOP/s on {cpu['tokens']} tokens; parity {cpu['parity_vs_gpu']}")

    line = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": kdtype,
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {spec.num_seqs} seq x {spec.q_per_seq} query tokens, {spec.num_heads} heads, "
                        f"top-{spec.topk} of a {spec.ctx}-token paged FP8 e4m3fn latent cache (page {spec.page_size}), "
                        f"qk 576 / v 512, scale_block_size {spec.scale_block_size}, sink {spec.sink}",
            "tokens": spec.num_tokens, "heads": spec.num_heads, "topk": spec.topk,
            "flop_per_call": flops, "flop_count": "2*H*(576+512) per gathered key",
            "num_splits": splits,
            "variant": args.variant,
            "cold_ms_per_call": cold_ms,
            "settle": {"calls": settle_calls, "ms": settle_ms},
        },
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": tflops / peak,
            "traffic": measured_traffic(args.workload, args.variant),
            "kernel": kname,
            "issued_mfma_frac": issued * tflops / peak,
            # the other roof: algorithmic HBM bytes per call (gathered rows
            # counted only when the pool exceeds the cache) and the rate at
            # which the listed rows reach LDS
            "hbm_bytes": hbm_bytes,
            "hbm_GBps": hbm_gbps,
            "hbm_frac": hbm_gbps / PEAK_HBM_GBPS,
            "gather_GBps": gathered / (ms * 1e-3) / 1e9,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
