#!/usr/bin/env python3
"""Benchmark of the fused inference attention hot path on one MI355X.

Prints ONE JSON line.  The headline workload is the causal GQA prefill
(B=4, Q_N=32, KV_N=8, D=128, bf16, per-batch lengths in [512, 2048]); a step
is one run of its plan (fia_run: the prefill kernel).  `value` is its
algorithmic TFLOP/s (visible (i, j) pairs only, 4*D flops per pair and head)
over the K timed steps.  The same line carries, as `components`, the other
hot-path workloads measured the same way: paged GQA decode (HBM GB/s), long
causal ALiBi prefill (TFLOP/s) and shared-KV sparse decode (GB/s).

Kernel durations come from HIP events recorded on the launch stream around
each run; `roofline` relates them to MI355X's published peaks.  The
`cpu_baseline` times the float64 oracle on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
SEEDS_HCA = 1006


def visible_pairs(mode, Lq, Lk):
    """Number of visible (i, j) pairs of one head for mask modes 0 / 2 / 3."""
    if mode == 0:
        return Lq * Lk
    total = 0
    d = Lk - Lq if mode == 3 else 0
    # row i sees keys j <= i + d, clipped to [0, Lk)
    for i in range(Lq):
        total += max(0, min(Lk, i + d + 1))
    return total


def dense_flops(case):
    B = case.batch
    lq = case.actual_seq_lengths or [case.q.shape[1]] * B
    lk = case.actual_seq_lengths_kv or [case.k.shape[1]] * B
    m = getattr(case, "atten_mask", None)
    if m is not None and case.sparse_mode in (0, 1):
        # explicit mask: the unmasked pairs of each batch's [Lq, Lk] corner
        m3 = m.reshape(-1, m.shape[-2], m.shape[-1])
        pairs = sum(int((m3[b if m3.shape[0] > 1 else 0, :int(a), :int(c)] == 0).sum())
                    for b, (a, c) in enumerate(zip(lq, lk)))
    else:
        pairs = sum(visible_pairs(case.sparse_mode, int(a), int(b)) for a, b in zip(lq, lk))
    return 4.0 * case.q.shape[-1] * case.num_heads * pairs


def decode_bytes(case):
    """Algorithmic HBM bytes of a paged decode: every visible K and V row once
    per KV head, plus Q, O, LSE and the block-table entries used."""
    D, kvn, qn = case.q.shape[-1], case.num_kv_heads, case.num_heads
    B = case.q.shape[0]
    L = case.actual_seq_lengths_kv
    aq = getattr(case, "kv_quant", None)
    if aq is None:
        kv = sum(L) * kvn * D * 2 * 2
    else:
        # one byte per code; per-token tables are read once per visible key
        # (shared by the KV heads), per-channel tables once
        kv = sum(L) * kvn * D * 2
        for mode, sc, of in ((aq["kmode"], aq["kscale"], aq["koff"]), (aq["vmode"], aq["vscale"], aq["voff"])):
            per = (sum(L) * 4) if mode == 1 else sc.nbytes
            kv += per * (2 if of is not None else 1)
    q = B * qn * D * 2
    o = q
    lse = B * qn * 4 if case.lse else 0
    bt = sum(-(-x // case.block_size) for x in L) * 4
    return kv + q + o + lse + bt


def sparse_bytes(case):
    """Selected rows at 604 used bytes each, q, out, indices (BSND or TND)."""
    N1, D = case.q.shape[-2], case.q.shape[-1]
    B = len(case.seqused_kv)
    if case.cu_seqlens_q is None:
        S1 = case.q.shape[1]
        counts = [S1] * B
        key = lambda b, t: (b, t)
    else:
        cu = case.cu_seqlens_q
        counts = [cu[b + 1] - cu[b] for b in range(B)]
        key = lambda b, t: cu[b] + t
    n_q = sum(counts)
    rows = 0
    for b, Lk in enumerate(case.seqused_kv):
        S1 = counts[b]
        for t in range(S1):
            p = Lk - S1 + t
            win = max(0, min(Lk - 1, p + case.win_right) - max(0, p - case.win_left) + 1)
            n_cmp = max(0, Lk // case.cmp_ratio - (S1 - 1 - t))
            if case.cmp_sparse_indices is None:     # heavily compressed: every visible row
                rows += win + n_cmp
            else:
                idx = case.cmp_sparse_indices[key(b, t)][0]
                rows += win + int(((idx >= 0) & (idx < n_cmp)).sum())
    idx_bytes = 0 if case.cmp_sparse_indices is None else case.cmp_sparse_indices.nbytes
    return rows * 604 + 2 * n_q * N1 * D * 2 + idx_bytes + (4 * (B + 1) if case.cu_seqlens_q else 0)


def time_plan(plan, steps, warmup, flush=None):
    """Run warmup untimed, then `steps` timed runs.  Returns (wall ms per
    step, mean device ms per run from HIP events on the launch stream).

    Without `flush` the runs go back to back between one pair of events, so
    the per-run figure carries no event overhead.  With `flush` (a cache
    scrub between runs, for working sets that fit in the caches) every run
    is bracketed by its own events and the wall figure is not taken."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        plan.run(stream)
    torch.cuda.synchronize()
    if flush is None:
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(steps):
            plan.run(stream)
        end.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1000.0 / steps
        return wall_ms, start.elapsed_time(end) / steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        flush()
        starts[k].record(stream)
        plan.run(stream)
        ends[k].record(stream)
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return None, sum(per) / len(per)


def per_launch(plan, launches, flush, flops):
    """Each launch bracketed by its own HIP events after a 512 MiB cache scrub
    (the working set then comes from HBM, not from the 256 MB last-level
    cache): median and min kernel time, and the rates they give."""
    import statistics
    import torch

    stream = torch.cuda.current_stream()
    plan.run(stream)
    ms = []
    for _ in range(launches):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        plan.run(stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    med, mn = statistics.median(ms), min(ms)
    return {"launches": launches, "median_ms": round(med, 5), "min_ms": round(mn, 5),
            "median_tflops": round(flops / (med / 1000.0) / 1e12, 3),
            "best_tflops": round(flops / (mn / 1000.0) / 1e12, 3),
            "cache": "512 MiB scrub before each launch"}


def kernel_source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_online_softmax_flash_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counts, scaled by the copy-kernel calibration; None when no counts were
    taken for the current kernel source."""
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(kernel)
    if not entry:
        return None
    if entry.get("source_digest") != kernel_source_digest(entry.get("sources", [])):
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(case, flops):
    from oracle import fia_oracle as O

    threads = None
    try:
        import threadpoolctl

        threads = sum(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
                      if i.get("user_api") == "blas") or None
    except Exception:
        pass
    # Whole passes of the oracle over the workload until at least 10 s of CPU
    # work (at most 30 passes), so the figure is not a one-shot timing.
    t0 = time.perf_counter()
    passes = 0
    while True:
        O.fia_case(case)
        passes += 1
        secs = time.perf_counter() - t0
        if secs >= 10.0 or passes >= 30:
            break
    return {"value": passes * flops / secs / 1e12, "unit": "TFLOP/s",
            "cores": threads or os.cpu_count(), "kind": "oracle", "seconds": round(secs, 3),
            "sample": f"{passes} whole passes of the causal GQA prefill workload (4 batches x 32 "
                      "heads), float64 numpy with materialised scores"}


def measure_peaks(dev):
    """Rates measured on this machine (the second roofline denominators):
    a loop of independent bf16 MFMAs on register operands, and a streaming
    read of a 2 GiB device buffer with 16-byte non-temporal loads; each the
    best of 5 timed launches after one warm-up."""
    import torch

    from attention_online_softmax_flash_amd import fia

    L = fia.lib()
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    n_wg, iters = 2048, 2000                  # 8 waves per CU, 2 per SIMD
    out = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    buf = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    out32 = torch.empty(4096 * 256, dtype=torch.int32, device=dev)

    def best(launch):
        launch()
        ms = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            b.record(stream)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return min(ms)

    def mfma():
        fia._check(L.fia_peak_mfma_bf16(n_wg, iters, out.data_ptr(), h))

    def read():
        fia._check(L.fia_peak_hbm_read(buf.data_ptr(), buf.numel(), 4096, out32.data_ptr(), h))

    t_mfma = best(mfma)
    t_read = best(read)
    flops = n_wg * 4 * iters * 8 * 32768
    res = {"mfma_bf16_tflops": round(flops / (t_mfma / 1e3) / 1e12, 1),
           "hbm_read_gbs": round(buf.numel() / (t_read / 1e3) / 1e9, 1),
           "how": "fia_peak_mfma_bf16 (2048 workgroups x 4 waves, 2000 iterations of 8 independent "
                  "32x32x16 bf16 MFMAs on registers) and fia_peak_hbm_read (2 GiB read once with "
                  "16-byte non-temporal loads, 4096 workgroups taking contiguous 32 KiB blocks, 8 loads in flight per thread); best of 5 launches"}
    del out, buf, out32
    return res


def add_measured_fracs(line, peaks):
    """Beside each roofline's fraction of the published peak, its fraction of
    the rate measured on this machine."""
    def one(r):
        if r is None:
            return
        m = peaks["mfma_bf16_tflops"] if r["unit"] == "TFLOP/s" else peaks["hbm_read_gbs"]
        r["measured_peak"] = m
        r["frac_measured"] = round(r["achieved"] / m, 4)
    one(line.get("roofline"))
    for c in line.get("components", {}).values():
        one(c.get("roofline"))


def progress(what):
    """One line on stderr per workload, so a long run shows it is alive."""
    print(f"[bench] {what} ...", file=sys.stderr, flush=True)


def roofline(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["all", "c1", "c2", "c3", "c4", "c5", "next", "c3q", "copy", "peaks"],
                    default="all",
                    help="limit the run to one workload (profiling); 'copy' runs a plain 1 GiB "
                         "device copy, the calibration of the HBM traffic counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator shards by batch / KV head with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from attention_online_softmax_flash_amd import torch_io as TI
    from attention_online_softmax_flash_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    if args.workload == "copy":
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                          "launches": 3}), flush=True)
        return
    want = lambda w: args.workload in ("all", w)
    flush_buf = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.zero_()
    components = {}
    line = None

    peaks = None
    if args.workload in ("all", "peaks"):
        progress("peaks")
        peaks = measure_peaks(dev)

    if want("c2"):
        progress("c2")
        case = W.c2_causal_gqa()
        flops = dense_flops(case)
        t0 = time.perf_counter()
        tensors = TI.dense_tensors(case, dev)
        t_plan = time.perf_counter()
        plan = TI.dense_plan(case, dev, tensors=tensors)
        plan_ms = (time.perf_counter() - t_plan) * 1000.0
        wall_ms, kern_ms = time_plan(plan, args.steps, args.warmup)
        value = flops / (wall_ms / 1000.0) / 1e12
        achieved = flops / (kern_ms / 1000.0) / 1e12
        line = {
            "metric": "decode attention HBM GB/s + prefill attention TFLOP/s, bf16, 1 MI355X",
            "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(wall_ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "causal GQA prefill: B=4, Q_N=32, KV_N=8, D=128, S padded "
                                   "to 2048, actual lengths " + str(case.actual_seq_lengths) +
                                   ", right-down causal, scale 1/sqrt(128)",
                       "global_batch": 4, "seq_len": 2048, "parallelism": "none",
                       "algorithmic_flop_per_step": flops, "plan_ms": round(plan_ms, 3)},
            "roofline": roofline("mfma", achieved, PEAK_BF16_TFLOPS, "TFLOP/s",
                                 measured_traffic("prefill_bf16")),
        }
        line["roofline"]["kernel"] = "prefill_bf16<128, false>"
        line["roofline"]["kernel_ms"] = round(kern_ms, 5)
        line["per_launch"] = per_launch(plan, max(20, args.steps), flush, flops)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(case, flops)
        del plan, tensors

    if want("c3"):
        progress("c3")
        case = W.c3_paged_decode()
        nbytes = decode_bytes(case)
        plan = TI.dense_plan(case, dev)
        # The KV cache (1.1 GB) is far larger than the L2 and last-level
        # caches, so back-to-back runs stream it from HBM every time.
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup)
        gbs = nbytes / (kern_ms / 1000.0) / 1e9
        components["paged_decode"] = {
            "workload": "paged GQA decode: B=64, Q_N=32, KV_N=8, D=128, block 128, KV lengths "
                        "in [1024, 8192], LSE", "unit": "GB/s", "value": round(gbs, 2),
            "algorithmic_bytes": nbytes, "ms": round(kern_ms, 5),
            "kernels": "decode_split_bf16<128> + decode_merge<128>",
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                 measured_traffic("decode_split_bf16"))}
        del plan
        # The same cache stored BnNBsD: each KV head's rows of a page contiguous.
        case_b = W.as_bnnbsd(case)
        plan = TI.dense_plan(case_b, dev)
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup)
        gbs = nbytes / (kern_ms / 1000.0) / 1e9
        components["paged_decode_bnnbsd"] = {
            "workload": "the paged GQA decode above with the KV pools in BnNBsD order "
                        "[n_blocks, KV_N, 128, D]", "unit": "GB/s", "value": round(gbs, 2),
            "algorithmic_bytes": nbytes, "ms": round(kern_ms, 5),
            "kernels": "decode_split_bf16<128> + decode_merge<128>",
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}
        del plan, case_b
        # The same decode with the KV lengths on the device: the partitioner
        # kernel builds the chunk list on every run, the grid is sized for
        # the 8192 bound.
        lens_dev = torch.tensor(case.actual_seq_lengths_kv, dtype=torch.int32, device=dev)
        plan = TI.dense_plan(case, dev, actual_seq_lengths_kv=None,
                             actual_seq_lengths_kv_device=lens_dev, max_actual_seq_length_kv=8192)
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup)
        gbs = nbytes / (kern_ms / 1000.0) / 1e9
        components["paged_decode_device_lengths"] = {
            "workload": "the paged GQA decode above with its KV lengths on the device (int32 [64]), "
                        "plan bound 8192", "unit": "GB/s", "value": round(gbs, 2),
            "algorithmic_bytes": nbytes, "ms": round(kern_ms, 5),
            "kernels": "decode_partition + decode_split_bf16<128> + decode_merge<128>",
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}
        del plan, lens_dev

    if want("c1"):
        progress("c1")
        # Correctness-sized fp32 workload: kernel time only (launch-bound; its
        # accuracy against the oracle is checked by the tests).
        case = W.c1_tiny_dense()
        plan = TI.dense_plan(case, dev)
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup)
        components["tiny_dense_fp32"] = {
            "workload": "tiny dense attention: B=1, N=2, S1=S2=64, D=64, fp32, no mask, LSE",
            "unit": "us", "value": round(kern_ms * 1000.0, 2), "kernels": "attn_fp32",
            "algorithmic_flop": dense_flops(case)}
        del plan

    if want("c4"):
        progress("c4")
        case = W.c4_alibi_prefill()
        flops = dense_flops(case)
        plan = TI.dense_plan(case, dev)
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup)
        tf = flops / (kern_ms / 1000.0) / 1e12
        components["long_alibi_prefill"] = {
            "workload": "causal ALiBi prefill: B=1, Q_N=KV_N=16, S=8192, D=128",
            "unit": "TFLOP/s", "value": round(tf, 3), "algorithmic_flop": flops,
            "ms": round(kern_ms, 5), "kernels": "prefill_bf16<128, true>",
            "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", measured_traffic("prefill_bf16_alibi")),
            "per_launch": per_launch(plan, 20, flush, flops)}
        del plan

    if want("c5"):
        progress("c5")
        case = W.c5_sparse_sharedkv()
        nbytes = sparse_bytes(case)
        plan = TI.sparse_plan(case, dev)
        # 8 MB of rows would stay cached between runs: scrub the caches.
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup, flush=flush)
        gbs = nbytes / (kern_ms / 1000.0) / 1e9
        components["sparse_sharedkv_decode"] = {
            "workload": "shared-KV sparse decode: B=16, Q_N=64, D=512 (fp8 nope + bf16 rope), "
                        "window 128 + top-512 of ratio-4 compressed KV, sinks",
            "unit": "GB/s", "value": round(gbs, 2), "algorithmic_bytes": nbytes,
            "ms": round(kern_ms, 5), "kernels": "sparse_chunk + sparse_merge",
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}
        del plan

    if want("next"):
        progress("next")
        # The causal GQA prefill workload with the inputs of the mask / bias /
        # sink parameter groups, and the heavily compressed sparse mode.
        base = W.c2_causal_gqa()
        variants = [
            ("prefill_explicit_mask", W.with_random_mask(base, 41, p_masked=0.1, mode=0),
             "causal GQA prefill shapes, sparse_mode 0 with a uint8 mask [4, 2048, 2048] "
             "(10 % of keys masked out, every key of the actual lengths otherwise)"),
            ("prefill_pse_bias", W.with_random_bias(base, 42, per_batch=False),
             "causal GQA prefill with a bf16 pse_shift bias [1, 32, 2048, 2048]"),
            ("prefill_learnable_sink", W.with_random_sink(base, 43),
             "causal GQA prefill with a bf16 learnable sink [32]"),
        ]
        for key, case, text in variants:
            flops = dense_flops(case)
            plan = TI.dense_plan(case, dev)
            _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup)
            tf = flops / (kern_ms / 1000.0) / 1e12
            components[key] = {
                "workload": text, "unit": "TFLOP/s", "value": round(tf, 3),
                "algorithmic_flop": flops, "ms": round(kern_ms, 5),
                "kernels": "prefill_bf16<128, false, 0, true>" if key != "prefill_learnable_sink"
                           else "prefill_bf16<128, false, 0, false>",
                "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", None)}
            del plan, case
        case = W.sparse_case("hca", SEEDS_HCA, B=16, N1=64, seqused_kv=[16384] * 16,
                             materialise_all_ori=False, heavily_compressed=True)
        nbytes = sparse_bytes(case)
        plan = TI.sparse_plan(case, dev)
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup, flush=flush)
        gbs = nbytes / (kern_ms / 1000.0) / 1e9
        components["sparse_heavily_compressed"] = {
            "workload": "shared-KV sparse decode, heavily compressed: B=16, Q_N=64, D=512, "
                        "window 128 + every row of the ratio-128 compressed KV (128 rows), sinks",
            "unit": "GB/s", "value": round(gbs, 2), "algorithmic_bytes": nbytes,
            "ms": round(kern_ms, 5), "kernels": "sparse_chunk + sparse_merge",
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}
        del plan
        # Two query tokens per batch entry (speculative decoding) at the
        # shared-KV sparse decode shapes.
        case = W.sparse_case("s1_2", SEEDS_HCA + 1, B=16, N1=64, seqused_kv=[16384] * 16, K2=512,
                             S1=2, materialise_all_ori=False)
        nbytes = sparse_bytes(case)
        plan = TI.sparse_plan(case, dev)
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup, flush=flush)
        gbs = nbytes / (kern_ms / 1000.0) / 1e9
        components["sparse_two_query_tokens"] = {
            "workload": "shared-KV sparse attention, 2 query tokens per batch entry: B=16, Q_N=64, "
                        "D=512, window 128 + top-512 of ratio-4 compressed KV per token, sinks",
            "unit": "GB/s", "value": round(gbs, 2), "algorithmic_bytes": nbytes,
            "ms": round(kern_ms, 5), "kernels": "sparse_chunk + sparse_merge",
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}
        del plan
        # TND: ragged query-token counts (1..4 per batch entry, seeded) packed
        # into T1 rows, the row-to-entry map read from cu_seqlens_q on the device.
        counts = [int(x) for x in W.rng_for(SEEDS_HCA + 2).integers(1, 5, size=16)]
        case = W.sparse_tnd_case("tnd", SEEDS_HCA + 3, q_counts=counts, B=16, N1=64,
                                 seqused_kv=[16384] * 16, K2=512, materialise_all_ori=False)
        nbytes = sparse_bytes(case)
        plan = TI.sparse_plan(case, dev)
        _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup, flush=flush)
        gbs = nbytes / (kern_ms / 1000.0) / 1e9
        components["sparse_tnd_ragged"] = {
            "workload": f"shared-KV sparse attention, TND with query counts {counts} (T1 = {sum(counts)}): "
                        "Q_N=64, D=512, window 128 + top-512 of ratio-4 compressed KV per token, sinks",
            "unit": "GB/s", "value": round(gbs, 2), "algorithmic_bytes": nbytes,
            "ms": round(kern_ms, 5), "kernels": "sparse_chunk + sparse_merge",
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}
        del plan

    if want("c3q"):
        progress("c3q")
        # The paged GQA decode with a fake-quantised KV cache (one byte per
        # element): int8 codes with per-token scales and offsets, and e4m3fn
        # codes with per-channel scales.
        case = W.c3_paged_decode()
        for key, kind, km, off, bn in (("paged_decode_int8_per_token", "int8", 1, True, False),
                                       ("paged_decode_fp8_per_channel", "fp8", 0, False, False),
                                       ("paged_decode_int8_per_token_bnnbsd", "int8", 1, True, True)):
            qc = W.with_kv_quant(case, 1007, kind=kind, kmode=km, vmode=km, offsets=off)
            if bn:
                qc = W.as_bnnbsd(qc)
            nbytes = decode_bytes(qc)
            plan = TI.dense_plan(qc, dev)
            _, kern_ms = time_plan(plan, min(args.steps, 20), args.warmup)
            gbs = nbytes / (kern_ms / 1000.0) / 1e9
            what = ("int8 codes, per-token fp32 scales and offsets" if kind == "int8"
                    else "e4m3fn codes, per-channel bf16 scales")
            if bn:
                what += ", pools in BnNBsD order [n_blocks, KV_N, 128, D]"
            components[key] = {
                "workload": "the paged GQA decode above with a fake-quantised KV cache: " + what,
                "unit": "GB/s", "value": round(gbs, 2), "algorithmic_bytes": nbytes,
                "ms": round(kern_ms, 5), "kernels": "decode_split_q8<128> + decode_merge<128>",
                "tokens_per_s": round(case.q.shape[0] / (kern_ms / 1000.0), 1),
                "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", None)}
            del plan, qc
        del case

    if line is None:
        line = {"metric": "decode attention HBM GB/s + prefill attention TFLOP/s, bf16, 1 MI355X",
                "value": None, "unit": None, "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "note": f"partial run: --workload {args.workload}"}
    line["components"] = components
    if peaks is not None:
        line["measured_peaks"] = peaks
        add_measured_fracs(line, peaks)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
