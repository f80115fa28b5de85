#!/usr/bin/env python3
"""Benchmark of the fused inference attention hot path on one MI355X.

Prints ONE JSON line.  The headline workload is the causal GQA prefill
(B=4, Q_N=32, KV_N=8, D=128, bf16, per-batch lengths in [512, 2048]); a step
is one run of its plan (fia_run: the prefill kernel).  `value` is its
algorithmic TFLOP/s (visible (i, j) pairs only, 4*D flops per pair and head)
over the K timed steps, each step on one of several input replicas in turn
(together more than twice the 256 MB last-level cache, so every step reads
its inputs from HBM).  The same line carries, as `components`, the other
hot-path workloads: paged GQA decode (HBM GB/s), long causal ALiBi prefill
(TFLOP/s), shared-KV sparse decode over packed fp8 rows and over bf16 rows
(GB/s), and the mask / bias / sink / fake-quant / sparse-mode variants.

Kernel durations come from HIP events recorded on the launch stream;
`roofline` relates them to MI355X's published peaks (and `frac_measured` to
the peaks measured on the machine); `traffic` is the HBM bytes per run from
committed rocprofv3 FETCH_SIZE / WRITE_SIZE counts.  Every workload also
carries `cpu_baseline`: the float64 oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
    python bench.py --counters-from DIR     (no GPU: rebuild the counters file)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
METRIC = "decode attention HBM GB/s + prefill attention TFLOP/s, bf16, 1 MI355X"
LLC_BYTES = 256 << 20          # MI355X last-level (Infinity) cache


# ---------------------------------------------------------------------------
# Algorithmic work of each workload.
# ---------------------------------------------------------------------------
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


def dense_pairs(case):
    """Visible (i, j) pairs of one head, summed over the batch."""
    B = case.batch
    lq = case.actual_seq_lengths or [case.q.shape[1]] * B
    lk = case.actual_seq_lengths_kv or [case.k.shape[1]] * B
    m = getattr(case, "atten_mask", None)
    if m is not None and case.sparse_mode in (0, 1):
        # explicit mask: the unmasked pairs of each batch's [Lq, Lk] corner
        m3 = m.reshape(-1, m.shape[-2], m.shape[-1])
        return sum(int((m3[b if m3.shape[0] > 1 else 0, :int(a), :int(c)] == 0).sum())
                   for b, (a, c) in enumerate(zip(lq, lk)))
    return sum(visible_pairs(case.sparse_mode, int(a), int(b)) for a, b in zip(lq, lk))


def dense_flops(case):
    return 4.0 * case.q.shape[-1] * case.num_heads * dense_pairs(case)


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
    """Selected rows (604 used bytes of a packed fp8 row, 1024 of an fp16 /
    bf16 row), q, out, indices, LSE (BSND or TND)."""
    N1, D = case.q.shape[-2], case.q.shape[-1]
    B = len(case.seqused_kv)
    half = hasattr(case, "kv_layout")            # sparse_flash_mla rows
    row_bytes = 2 * D if half else 604
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
            if half and case.cmp_kv is None:
                rows += win
            elif case.cmp_sparse_indices is None:     # heavily compressed: every visible row
                rows += win + n_cmp
            else:
                idx = case.cmp_sparse_indices[key(b, t)][0]
                rows += win + int(((idx >= 0) & (idx < n_cmp)).sum())
    idx_bytes = 0 if case.cmp_sparse_indices is None else case.cmp_sparse_indices.nbytes
    lse = n_q * N1 * 4 if (half and case.return_lse) else 0
    return (rows * row_bytes + 2 * n_q * N1 * D * 2 + idx_bytes + lse +
            (4 * (B + 1) if case.cu_seqlens_q else 0))


# ---------------------------------------------------------------------------
# Timing.
# ---------------------------------------------------------------------------
def time_runs(plans, steps, warmup):
    """Run the plans round robin: `warmup` untimed runs, then `steps` timed
    runs back to back.  Returns (host wall ms per step, bracketed by device
    synchronisation, and device ms per step from HIP events on the launch
    stream)."""
    import torch

    stream = torch.cuda.current_stream()
    n = len(plans)
    for k in range(warmup):
        plans[k % n].run(stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(steps):
        plans[k % n].run(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0 / steps
    return wall_ms, start.elapsed_time(end) / steps


def time_scrubbed(plan, launches, flush):
    """Each launch bracketed by its own HIP events after a 512 MiB cache
    scrub: (mean, median, min) device ms."""
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
    return sum(ms) / len(ms), statistics.median(ms), min(ms)


def replicas_for(bytes_per_replica):
    """Input replicas needed so that the ones touched since a replica's last
    run exceed the last-level cache twice over."""
    return max(2, min(8, 1 + -(-2 * LLC_BYTES // max(1, bytes_per_replica))))


# ---------------------------------------------------------------------------
# HBM traffic counters and oracle timing.
# ---------------------------------------------------------------------------
def kernel_source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_online_softmax_flash_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(component):
    """HBM bytes per run of a component from committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE counts, scaled by the copy-kernel calibration; None when no
    counts were taken for the current kernel sources."""
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(component)
    if not entry:
        return None
    if entry.get("source_digest") != kernel_source_digest(entry.get("sources", [])):
        return None
    return entry.get("hbm_bytes_per_run")


def blas_threads():
    try:
        import threadpoolctl

        return sum(i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
                   if i.get("user_api") == "blas") or None
    except Exception:
        return None


def cpu_baseline(fn, work, unit, sample, min_seconds=8.0, max_passes=30):
    """The float64 oracle `fn` timed on the host cores: whole passes until at
    least `min_seconds` of CPU work; `work` is the algorithmic work of one
    pass in the unit's base quantity (flop or byte)."""
    t0 = time.perf_counter()
    passes = 0
    while True:
        fn()
        passes += 1
        secs = time.perf_counter() - t0
        if secs >= min_seconds or passes >= max_passes:
            break
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    return {"value": round(passes * work / secs / scale, 6), "unit": unit,
            "cores": os.cpu_count(), "blas_threads": blas_threads(), "kind": "oracle",
            "seconds": round(secs, 3), "passes": passes, "sample": sample}


def roofline(bound, achieved, peak, unit, traffic):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def progress(what):
    """One line on stderr per workload, so a long run shows it is alive."""
    print(f"[bench] {what} ...", file=sys.stderr, flush=True)


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
                  "16-byte non-temporal loads, 4096 workgroups taking contiguous 32 KiB blocks, 8 "
                  "loads in flight per thread); best of 5 launches"}
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
        one(c.get("roofline_bytes"))


# ---------------------------------------------------------------------------
# Workloads.  Each component builds its plans, times them and returns its
# JSON object; `ctx` carries the device, the step counts and the scrub.
# ---------------------------------------------------------------------------
class Ctx:
    def __init__(self, args, dev, flush):
        self.steps, self.warmup, self.cpu, self.dev, self.flush = (
            args.steps, args.warmup, not args.no_cpu_baseline, dev, flush)


def _mods():
    from attention_online_softmax_flash_amd import torch_io as TI
    from attention_online_softmax_flash_amd import workloads as W
    from oracle import fia_oracle as O
    return TI, W, O


def _input_bytes(tensors):
    return sum(t.numel() * t.element_size() for t in tensors if t is not None)


def prefill_component(ctx, case, key, workload, kernel, cpu_fn=None, cpu_work=None, cpu_sample=None,
                      extra_bytes=0):
    """A prefill workload: plans on rotating input replicas (cache-cold
    steps) plus one back-to-back figure on a single replica (warm)."""
    TI, W, O = _mods()
    flops = dense_flops(case)
    plans = [TI.dense_plan(case, ctx.dev)]
    per = _input_bytes([plans[0].query, plans[0].key, plans[0].value, plans[0].out,
                        plans[0].pse_shift, plans[0].atten_mask])
    for _ in range(replicas_for(per) - 1):
        plans.append(TI.dense_plan(case, ctx.dev))
    wall_ms, kern_ms = time_runs(plans, ctx.steps, ctx.warmup)
    _, warm_ms = time_runs(plans[:1], ctx.steps, ctx.warmup)
    tf = flops / (kern_ms / 1000.0) / 1e12
    out = {"workload": workload, "unit": "TFLOP/s", "value": round(tf, 3),
           "algorithmic_flop": flops, "ms": round(kern_ms, 5),
           "timing": f"{len(plans)} input replicas ({len(plans) * per / 2**20:.0f} MiB) run in turn, "
                     "back to back: every run reads its inputs from HBM",
           "warm_ms": round(warm_ms, 5), "warm_tflops": round(flops / (warm_ms / 1000.0) / 1e12, 3),
           "kernels": kernel,
           "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", measured_traffic(key))}
    if extra_bytes:
        # inputs streamed per visible pair (a mask or bias tensor): the byte
        # roofline beside the flop one
        gbs = extra_bytes / (kern_ms / 1000.0) / 1e9
        out["algorithmic_bytes"] = extra_bytes
        out["roofline_bytes"] = roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", measured_traffic(key))
    if ctx.cpu and cpu_fn is not None:
        out["cpu_baseline"] = cpu_baseline(cpu_fn, cpu_work, "TFLOP/s", cpu_sample)
    return out, wall_ms, plans


def comp_c2(ctx):
    TI, W, O = _mods()
    case = W.c2_causal_gqa()
    out, wall_ms, plans = prefill_component(
        ctx, case, "c2", "causal GQA prefill", "prefill_bf16<128, false, 0, false>",
        cpu_fn=lambda: O.fia_case(case), cpu_work=dense_flops(case),
        cpu_sample="whole passes of the causal GQA prefill workload (4 batches x 32 heads), "
                   "float64 numpy with materialised scores")
    out["wall_ms"] = round(wall_ms, 5)
    # per launch after a 512 MiB scrub (the previous round's headline protocol)
    mean, med, mn = time_scrubbed(plans[0], max(20, ctx.steps), ctx.flush)
    out["per_launch_scrubbed"] = {"median_ms": round(med, 5), "min_ms": round(mn, 5),
                                  "median_tflops": round(dense_flops(case) / (med / 1000) / 1e12, 3)}
    return out, case


def comp_c4(ctx):
    TI, W, O = _mods()
    case = W.c4_alibi_prefill()
    heads = [0, 1]
    out, _, _ = prefill_component(
        ctx, case, "c4", "long causal ALiBi prefill: B=1, Q_N=KV_N=16, S=8192, D=128",
        "prefill_bf16<128, true, 0, false>",
        cpu_fn=lambda: O.fia_case(case, heads=heads), cpu_work=dense_flops(case) * len(heads) / 16,
        cpu_sample="query heads 0 and 1 of the 16 (2 x 8192 rows, every key), float64 numpy with "
                   "materialised scores, whole passes")
    return out


def qkvo_bytes(case):
    """Query, key, value and output rows inside the actual lengths, once."""
    D, B = case.q.shape[-1], case.batch
    lq = case.actual_seq_lengths or [case.q.shape[1]] * B
    lk = case.actual_seq_lengths_kv or [case.k.shape[1]] * B
    return sum(2 * a * case.num_heads + 2 * c * case.num_kv_heads for a, c in zip(lq, lk)) * D * 2


def _prefill_variant(ctx, key, make, text, kernel, extra):
    TI, W, O = _mods()
    case = make()
    out, _, _ = prefill_component(
        ctx, case, key, text, kernel,
        cpu_fn=lambda: O.fia_case(case, heads=list(range(4))), cpu_work=dense_flops(case) * 4 / 32,
        cpu_sample="query heads 0-3 of the 32 (every batch and row), float64 numpy, whole passes",
        extra_bytes=(extra(case) + qkvo_bytes(case)) if extra else 0)
    return out


def comp_mask(ctx):
    TI, W, O = _mods()
    return _prefill_variant(
        ctx, "mask", W.mask_prefill,
        "causal GQA prefill shapes, sparse_mode 0 with a uint8 mask [4, 2048, 2048] (10 % of keys "
        "masked out, every key of the actual lengths otherwise)", "prefill_bf16<128, false, 0, true>",
        # one mask byte per (i, j) of every batch's [Lq, Lk] corner, shared by the heads
        lambda c: sum(a * a for a in c.actual_seq_lengths))


def comp_bias(ctx):
    TI, W, O = _mods()
    return _prefill_variant(
        ctx, "bias", W.bias_prefill,
        "causal GQA prefill with a bf16 pse_shift bias [1, 32, 2048, 2048]",
        "prefill_bf16<128, false, 0, true>",
        # 2 bytes of bias per visible (i, j) pair and query head; a bias
        # shared by the batch entries (leading dim 1) is read once, and the
        # causal corners of the shorter entries lie inside the longest one's
        lambda c: 2 * c.num_heads * (dense_pairs(c) if c.pse_bias.shape[0] > 1 else max(
            visible_pairs(c.sparse_mode, int(L), int(L)) for L in c.actual_seq_lengths)))


def comp_sink(ctx):
    TI, W, O = _mods()
    return _prefill_variant(ctx, "sink", W.sink_prefill,
                            "causal GQA prefill with a bf16 learnable sink [32]",
                            "prefill_bf16<128, false, 0, false>", None)


def decode_component(ctx, case, key, workload, kernels, plan_kw=None, cpu=True):
    TI, W, O = _mods()
    nbytes = decode_bytes(case)
    plan = TI.dense_plan(case, ctx.dev, **(plan_kw or {}))
    # The KV cache (>= 0.5 GB) is far larger than the last-level cache, so
    # back-to-back runs stream it from HBM every time.
    _, kern_ms = time_runs([plan], min(ctx.steps, 20), ctx.warmup)
    gbs = nbytes / (kern_ms / 1000.0) / 1e9
    out = {"workload": workload, "unit": "GB/s", "value": round(gbs, 2), "algorithmic_bytes": nbytes,
           "ms": round(kern_ms, 5), "kernels": kernels,
           "tokens_per_s": round(case.q.shape[0] / (kern_ms / 1000.0), 1),
           "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", measured_traffic(key))}
    if plan_kw is None:
        out["read_ceiling"] = read_ceiling(plan, case, kern_ms, ctx)
    if ctx.cpu and cpu:
        out["cpu_baseline"] = cpu_baseline(lambda: O.fia_case(case), nbytes, "GB/s",
                                           "whole passes of this decode workload (every batch and "
                                           "head), float64 numpy with materialised scores")
    del plan
    return out


def read_ceiling(plan, case, kern_ms, ctx):
    """The decode against a pure read of its own key / value rows
    (fia_debug_read_kv): the same rows, block-table lookups and request sizes,
    no arithmetic, timed back to back like the decode.  Order 0 reads one KV
    head's row per request (the decode kernels' order), order 1 a token's
    whole row of KV_N heads (where the pool keeps them adjacent)."""
    import torch

    stream = torch.cuda.current_stream()
    res = {"how": "fia_debug_read_kv, back to back; kv_bytes = every visible key and value row once"}
    L = case.actual_seq_lengths_kv
    esz = 1 if getattr(case, "kv_quant", None) else 2
    kv_bytes = sum(L) * case.num_kv_heads * case.q.shape[-1] * esz * 2
    res["kv_bytes"] = kv_bytes
    for order in (0, 1):
        try:
            out = plan.read_kv(order)
        except Exception as e:   # no instantiation for this shape / layout
            res[f"order{order}"] = f"n/a ({e.__class__.__name__})"
            continue
        n = min(ctx.steps, 20)
        for _ in range(ctx.warmup):
            plan.read_kv(order, out=out, stream=stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            plan.read_kv(order, out=out, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        res[f"order{order}"] = {"ms": round(ms, 5), "gbs": round(kv_bytes / (ms / 1000.0) / 1e9, 1),
                                "decode_vs_read": round(ms / kern_ms, 3)}
    return res


def comp_c3(ctx):
    TI, W, O = _mods()
    return decode_component(ctx, W.c3_paged_decode(), "c3",
                            "paged GQA decode: B=64, Q_N=32, KV_N=8, D=128, block 128, KV lengths "
                            "in [1024, 8192], LSE", "decode_split_bf16<128> + decode_merge<128>")


def comp_c3_bnnbsd(ctx):
    TI, W, O = _mods()
    return decode_component(ctx, W.as_bnnbsd(W.c3_paged_decode()), "c3_bnnbsd",
                            "the paged GQA decode with the KV pools in BnNBsD order "
                            "[n_blocks, KV_N, 128, D]", "decode_split_bf16<128> + decode_merge<128>",
                            cpu=False)


def comp_c3_devlen(ctx):
    import torch

    TI, W, O = _mods()
    case = W.c3_paged_decode()
    lens = torch.tensor(case.actual_seq_lengths_kv, dtype=torch.int32, device=ctx.dev)
    return decode_component(ctx, case, "c3_devlen",
                            "the paged GQA decode with its KV lengths on the device (int32 [64]), "
                            "plan bound 8192",
                            "decode_partition + decode_split_bf16<128> + decode_merge<128>",
                            plan_kw=dict(actual_seq_lengths_kv=None, actual_seq_lengths_kv_device=lens,
                                         max_actual_seq_length_kv=8192), cpu=False)


def _q8(ctx, key, kind, km, off, bn, text):
    TI, W, O = _mods()
    qc = W.q8_decode(key)
    return decode_component(ctx, qc, key, "the paged GQA decode with a fake-quantised KV cache: " + text,
                            "decode_split_q8<128> + decode_merge<128>", cpu=(key == "q8_int8"))


def comp_q8_int8(ctx):
    return _q8(ctx, "q8_int8", "int8", 1, True, False, "int8 codes, per-token fp32 scales and offsets")


def comp_q8_fp8(ctx):
    return _q8(ctx, "q8_fp8", "fp8", 0, False, False, "e4m3fn codes, per-channel bf16 scales")


def comp_q8_int8_bnnbsd(ctx):
    return _q8(ctx, "q8_int8_bnnbsd", "int8", 1, True, True,
               "int8 codes, per-token fp32 scales and offsets, pools in BnNBsD order")


def sparse_component(ctx, case, key, workload, cpu_fn=None, cpu_sample=None):
    """A sparse workload: each launch after a 512 MiB scrub (its few MB of
    rows would otherwise stay cached), plus the warm back-to-back figure."""
    TI, W, O = _mods()
    nbytes = sparse_bytes(case)
    half = hasattr(case, "kv_layout")
    plan = TI.sfmla_plan(case, ctx.dev) if half else TI.sparse_plan(case, ctx.dev)
    mean, med, mn = time_scrubbed(plan, max(20, ctx.steps), ctx.flush)
    _, warm_ms = time_runs([plan], ctx.steps, ctx.warmup)
    gbs = nbytes / (mean / 1000.0) / 1e9
    fmt = "1" if half else "0"
    out = {"workload": workload, "unit": "GB/s", "value": round(gbs, 2), "algorithmic_bytes": nbytes,
           "ms": round(mean, 5), "median_ms": round(med, 5), "min_ms": round(mn, 5),
           "timing": "each launch after a 512 MiB scrub (caches cold), HIP events around it",
           "warm_ms": round(warm_ms, 5),
           "kernels": f"sparse_attn<{fmt}> + sparse_merge",
           "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", measured_traffic(key))}
    if ctx.cpu and cpu_fn is not None:
        out["cpu_baseline"] = cpu_baseline(cpu_fn, nbytes, "GB/s", cpu_sample)
    del plan
    return out


def comp_c5(ctx):
    TI, W, O = _mods()
    case = W.c5_sparse_sharedkv()
    return sparse_component(ctx, case, "c5",
                            "shared-KV sparse decode: B=16, Q_N=64, D=512 (fp8 nope + bf16 rope), "
                            "window 128 + top-512 of ratio-4 compressed KV, sinks",
                            cpu_fn=lambda: O.sparse_sharedkv(case),
                            cpu_sample="whole passes of this workload, float64 numpy")


def comp_sfmla(ctx):
    TI, W, O = _mods()
    case = W.sfmla_decode_bf16()
    return sparse_component(ctx, case, "sfmla",
                            "sparse_flash_mla decode over bf16 rows: B=16, Q_N=64, D=512, window 128 "
                            "+ top-512 of ratio-4 compressed KV, PA_BBND block 128, sinks, LSE",
                            cpu_fn=lambda: O.sparse_flash_mla(case),
                            cpu_sample="whole passes of this workload, float64 numpy")


def comp_hca(ctx):
    TI, W, O = _mods()
    case = W.sparse_hca_decode()
    return sparse_component(ctx, case, "hca",
                            "shared-KV sparse decode, heavily compressed: B=16, Q_N=64, D=512, window "
                            "128 + every row of the ratio-128 compressed KV (128 rows), sinks")


def comp_s1_2(ctx):
    TI, W, O = _mods()
    case = W.sparse_two_tokens()
    return sparse_component(ctx, case, "s1_2",
                            "shared-KV sparse attention, 2 query tokens per batch entry: B=16, Q_N=64, "
                            "D=512, window 128 + top-512 of ratio-4 compressed KV per token, sinks")


def comp_tnd(ctx):
    TI, W, O = _mods()
    counts = W.sparse_tnd_counts()
    case = W.sparse_tnd_ragged()
    return sparse_component(ctx, case, "tnd",
                            f"shared-KV sparse attention, TND with query counts {counts} "
                            f"(T1 = {sum(counts)}): Q_N=64, D=512, window 128 + top-512 of ratio-4 "
                            "compressed KV per token, sinks")


def comp_c1(ctx):
    TI, W, O = _mods()
    # Correctness-sized fp32 workload: kernel time only (launch-bound; its
    # accuracy against the oracle is checked by the tests).
    case = W.c1_tiny_dense()
    plan = TI.dense_plan(case, ctx.dev)
    _, kern_ms = time_runs([plan], min(ctx.steps, 20), ctx.warmup)
    return {"workload": "tiny dense attention: B=1, N=2, S1=S2=64, D=64, fp32, no mask, LSE",
            "unit": "us", "value": round(kern_ms * 1000.0, 2), "kernels": "attn_fp32",
            "algorithmic_flop": dense_flops(case)}


COMPONENTS = {
    "c3": ("paged_decode", comp_c3),
    "c3_bnnbsd": ("paged_decode_bnnbsd", comp_c3_bnnbsd),
    "c3_devlen": ("paged_decode_device_lengths", comp_c3_devlen),
    "c1": ("tiny_dense_fp32", comp_c1),
    "c4": ("long_alibi_prefill", comp_c4),
    "c5": ("sparse_sharedkv_decode", comp_c5),
    "sfmla": ("sparse_flash_mla_decode_bf16", comp_sfmla),
    "mask": ("prefill_explicit_mask", comp_mask),
    "bias": ("prefill_pse_bias", comp_bias),
    "sink": ("prefill_learnable_sink", comp_sink),
    "hca": ("sparse_heavily_compressed", comp_hca),
    "s1_2": ("sparse_two_query_tokens", comp_s1_2),
    "tnd": ("sparse_tnd_ragged", comp_tnd),
    "q8_int8": ("paged_decode_int8_per_token", comp_q8_int8),
    "q8_fp8": ("paged_decode_fp8_per_channel", comp_q8_fp8),
    "q8_int8_bnnbsd": ("paged_decode_int8_per_token_bnnbsd", comp_q8_int8_bnnbsd),
}
GROUPS = {
    "all": ["c2"] + list(COMPONENTS),
    "c3all": ["c3", "c3_bnnbsd", "c3_devlen"],
    "next": ["mask", "bias", "sink", "hca", "s1_2", "tnd"],
    "c3q": ["q8_int8", "q8_fp8", "q8_int8_bnnbsd"],
}

# Kernels and sources of each component, for the counters file.
PRE_SRC = ["prefill.hip", "fia_device.h", "fia_internal.h"]
DEC_SRC = ["decode.hip", "fia_device.h", "fia_internal.h"]
Q8_SRC = ["decode_q8.hip", "decode.hip", "fia_device.h", "fia_internal.h"]
SP_SRC = ["sparse.hip", "fia_device.h", "fia_internal.h"]
COUNTER_KERNELS = {
    "c2": (PRE_SRC, ["prefill_bf16<"]),
    "c4": (PRE_SRC, ["prefill_bf16<"]),
    "mask": (PRE_SRC, ["prefill_bf16<"]),
    "bias": (PRE_SRC, ["prefill_bf16<"]),
    "sink": (PRE_SRC, ["prefill_bf16<"]),
    "c3": (DEC_SRC, ["decode_split_bf16", "decode_merge"]),
    "c3_bnnbsd": (DEC_SRC, ["decode_split_bf16", "decode_merge"]),
    "c3_devlen": (DEC_SRC, ["decode_partition", "decode_split_bf16", "decode_merge"]),
    "q8_int8": (Q8_SRC, ["decode_split_q8", "decode_merge"]),
    "q8_fp8": (Q8_SRC, ["decode_split_q8", "decode_merge"]),
    "q8_int8_bnnbsd": (Q8_SRC, ["decode_split_q8", "decode_merge"]),
    "c5": (SP_SRC, ["sparse_attn", "sparse_merge"]),
    "sfmla": (SP_SRC, ["sparse_attn", "sparse_merge"]),
    "hca": (SP_SRC, ["sparse_attn", "sparse_merge"]),
    "s1_2": (SP_SRC, ["sparse_attn", "sparse_merge"]),
    "tnd": (SP_SRC, ["sparse_attn", "sparse_merge"]),
}


def counters_from(d):
    """Rebuild profiles/hbm_counters.json from rocprofv3 --pmc runs under `d`:
    d/pmc_<component>_<FETCH_SIZE|WRITE_SIZE>/ (one counter per run of
    `bench.py --workload <component>`) and d/pmc_copy_* (the calibration:
    `bench.py --workload copy`, a plain 1 GiB device copy)."""
    import collections
    import csv

    def per_dispatch(comp, counter):
        files = glob.glob(os.path.join(d, f"pmc_{comp}_{counter}", "**", "*counter_collection.csv"),
                          recursive=True)
        if not files:
            return None
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in csv.DictReader(open(files[0])):
            acc[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: sum(v.values()) / len(v) for k, v in acc.items()}

    def pick(table, sub):
        hits = [v for k, v in table.items() if sub in k]
        return hits[0] if hits else None

    cf = pick(per_dispatch("copy", "FETCH_SIZE"), "copyBuffer")
    cw = pick(per_dispatch("copy", "WRITE_SIZE"), "copyBuffer")
    fs, ws = round(1048576.0 / cf, 4), round(1048576.0 / cw, 4)
    out = {"_calibration": {
        "copy_bytes": 1 << 30, "fetch_kib_per_copy": round(cf, 1), "write_kib_per_copy": round(cw, 1),
        "fetch_scale": fs, "write_scale": ws,
        "note": "a plain 1 GiB device copy (bench.py --workload copy) reads and writes 1 GiB; "
                "each kernel's FETCH_SIZE / WRITE_SIZE KiB per dispatch is scaled by the copy's "
                "factors"}}
    for comp, (src, kernels) in COUNTER_KERNELS.items():
        fetch, write = per_dispatch(comp, "FETCH_SIZE"), per_dispatch(comp, "WRITE_SIZE")
        if not fetch or not write:
            continue
        ks, total = {}, 0.0
        for sub in kernels:
            f, w = pick(fetch, sub), pick(write, sub)
            if f is None or w is None:
                continue
            ks[sub] = {"fetch_kib_per_dispatch": round(f, 1), "write_kib_per_dispatch": round(w, 1)}
            total += (f * fs + w * ws) * 1024
        out[comp] = {"sources": src, "source_digest": kernel_source_digest(src), "kernels": ks,
                     "hbm_bytes_per_run": int(round(total))}
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "c2", "copy", "peaks"] + list(GROUPS) + list(COMPONENTS),
                    help="limit the run to one workload or group (profiling); 'copy' runs a plain "
                         "1 GiB device copy, the calibration of the HBM traffic counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters-from", metavar="DIR",
                    help="rebuild profiles/hbm_counters.json from rocprofv3 --pmc output in DIR")
    args = ap.parse_args()
    if args.counters_from:
        res = counters_from(args.counters_from)
        print(json.dumps({k: v.get("hbm_bytes_per_run", v.get("fetch_scale")) for k, v in res.items()}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator shards by batch / KV head with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch

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
    names = GROUPS.get(args.workload, [args.workload])
    flush_buf = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.zero_()
    ctx = Ctx(args, dev, flush)
    components = {}
    line = None

    peaks = None
    if args.workload in ("all", "peaks"):
        progress("peaks")
        peaks = measure_peaks(dev)

    if "c2" in names:
        progress("c2")
        c2, case = comp_c2(ctx)
        flops = c2["algorithmic_flop"]
        wall_ms = c2["wall_ms"]
        line = {
            "metric": METRIC, "value": round(flops / (wall_ms / 1000.0) / 1e12, 3), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "causal GQA prefill: B=4, Q_N=32, KV_N=8, D=128, S padded to 2048, "
                                   "actual lengths " + str(case.actual_seq_lengths) +
                                   ", right-down causal, scale 1/sqrt(128)",
                       "global_batch": 4, "seq_len": 2048, "parallelism": "none",
                       "algorithmic_flop_per_step": flops, "timing": c2["timing"]},
            "roofline": dict(c2["roofline"], kernel="prefill_bf16<128, false>",
                             kernel_ms=c2["ms"]),
            "warm_back_to_back": {"ms": c2["warm_ms"], "tflops": c2["warm_tflops"]},
            "per_launch_scrubbed": c2["per_launch_scrubbed"],
        }
        if "cpu_baseline" in c2:
            line["cpu_baseline"] = c2["cpu_baseline"]
    for n in names:
        if n == "c2":
            continue
        key, fn = COMPONENTS[n]
        progress(n)
        components[key] = fn(ctx)
        torch.cuda.empty_cache()

    if line is None:
        line = {"metric": METRIC, "value": None, "unit": None, "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "note": f"partial run: --workload {args.workload}"}
    line["components"] = components
    if peaks is not None:
        line["measured_peaks"] = peaks
        add_measured_fracs(line, peaks)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
