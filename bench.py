"""FlashAttention forward + backward throughput on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
fa_fwd (O in the input dtype, lse), then the backward's two stages
(fa_bwd_dq_and_stats -> fa_bwd_dkdv, exactly what fa_bwd runs), all through
the library's C ABI on torch's current stream.

Default workload: Z=128, H=8, N=1024, D=128, fp16, causal, scale=1/sqrt(128)
(seeded i.i.d. N(0,1) Q/K/V/dO).  Prints ONE JSON line with:
  value       fwd+bwd TFLOP/s (FlashAttention convention: fwd = 4 Z H N^2 D,
              halved when causal; bwd = 2.5 x fwd)
  breakdown   fwd, bwd and per-kernel times, TFLOP/s and fraction of peak
  roofline    the kernel taking most of the step, against its own bound
  cpu_baseline the fp64 oracle on a bounded sample of the same workload

Kernel durations come from HIP events recorded between the stage calls on the
stream the kernels run on, inside the timed region.  Inputs are resident in
HBM before timing starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402  (seeded inputs only; no attention arithmetic)

# MI355X published dense peaks.
PEAK_MFMA_F16_TFLOPS = 2516.6   # fp16 / bf16 dense MFMA
PEAK_HBM_GBS = 8000.0           # HBM3E
DEFAULT_WORKLOAD = "d128_causal"
KERNELS = ("fa_fwd", "fa_bwd_dq", "fa_bwd_dkdv")  # the step, in launch order
# The step with the fused per-head backward: statistics pass, then one pass for dQ, dK, dV.
KERNELS_FUSED = ("fa_fwd", "fa_bwd_pre", "fa_bwd_fused")
# Source files each kernel is built from; a stored traffic measurement is only
# reported while these are unchanged.
KERNEL_SOURCES = {
    "fa_fwd": ("fa_fwd.hip", "fa_device.h", "fa_kernels.h", "fa_schedule.h"),
    "fa_bwd_pre": ("fa_bwd.hip", "fa_device.h", "fa_kernels.h"),
    "fa_bwd_dkdv": ("fa_bwd.hip", "fa_device.h", "fa_kernels.h", "fa_schedule.h"),
    "fa_bwd_dq": ("fa_bwd.hip", "fa_device.h", "fa_kernels.h", "fa_schedule.h"),
    "fa_bwd_fused": ("fa_bwd_fused.hip", "fa_device.h", "fa_kernels.h", "fa_schedule.h"),
    "fa_paged_decode": ("fa_paged.hip", "fa_device.h", "fa_kernels.h"),
    "fa_paged_decode_sparse": ("fa_paged.hip", "fa_device.h", "fa_kernels.h"),
    "fa_paged_decode_sources": ("fa_paged.hip", "fa_device.h", "fa_kernels.h"),
    "fa_paged_attention_sources": ("fa_paged.hip", "fa_device.h", "fa_kernels.h"),
    "fa_quest_select": ("fa_quest.hip", "fa_device.h", "fa_kernels.h"),
}


def fwd_flops(w) -> float:
    """4 N^2 D per (sequence, query head), halved when causal; a variable-length
    batch sums over its sequences."""
    if w.varlen:
        f = 4.0 * w.H * w.D * float(sum(n * n for n in w.lengths))
    else:
        f = 4.0 * w.Z * w.H * w.N * w.N * w.D
    return f / 2 if w.causal else f


def kernel_work(w, o_bytes: int):
    """Algorithmic work of one launch of each kernel: (bound, amount, unit).

    fa_fwd: the two forward GEMMs (QK^T, PV), 4 N^2 D per head (x 1/2 causal).
    fa_bwd_dkdv: four of the five counted backward GEMMs (QK^T recompute,
      dO V^T, P^T dO, dS^T Q), 8 N^2 D per head (x 1/2 causal).
    fa_bwd_dq: the fifth (dS K), 2 N^2 D per head (x 1/2 causal); its two
      recomputed GEMMs, and the row statistics (Delta, lse * log2 e) it
      computes for the dK/dV pass, are not counted.
    fa_bwd_pre (the standalone statistics pass, not part of the step): HBM
      bytes, read O and dO rows and lse, write two fp32 per row.
    """
    hf = fwd_flops(w)  # = 4 N^2 D per head, halved when causal
    rows = w.H * w.T if w.varlen else w.Z * w.H * w.N
    return {
        "fa_fwd": ("mfma", hf, "flop"),
        "fa_bwd_fused": ("mfma", 2.5 * hf, "flop"),
        "fa_bwd_dkdv": ("mfma", 2.0 * hf, "flop"),
        "fa_bwd_dq": ("mfma", 0.5 * hf, "flop"),
        "fa_bwd_pre": ("hbm", float(rows * (w.D * o_bytes + w.D * 2 + 12)), "byte"),
    }


def _computed_pairs(n: int, bq: int, bk: int, causal: bool) -> int:
    """(query, key) pairs a kernel computes for one head of n tokens when it
    works in blocks of bq queries x bk keys and, with the causal mask, skips
    only the blocks whose keys all follow the block's last query."""
    n_kt = -(-n // bk)
    total = 0
    for q0 in range(0, n, bq):
        nt = min((q0 + bq - 1) // bk + 1, n_kt) if causal else n_kt
        total += bq * bk * nt
    return total


def executed_over_counted(w) -> dict:
    """Matrix work each kernel executes over the work it is credited with.

    fa_fwd: 32-query blocks (one per wave) x key tiles of 64 (D = 64) or 32
      keys; at D = 256 both waves of a pair run the score product (1.5x).
    fa_bwd_dq: the same blocks, three products (S, dP recomputed; dS K) for
      the one counted.
    fa_bwd_dkdv: 32-key x 32-query blocks, the four counted products.
    Counted pairs are n^2 (n^2 / 2 causal), as in the FLOP convention."""
    lengths = list(w.lengths) if w.varlen else [w.N]
    bk = 64 if w.D == 64 else 32
    counted = sum(n * n / (2 if w.causal else 1) for n in lengths)
    fwd = sum(_computed_pairs(n, 32, bk, w.causal) for n in lengths) / counted
    dkdv = sum(_computed_pairs(n, 32, 32, w.causal) for n in lengths) / counted
    return {"fa_fwd": round(fwd * (1.5 if w.D == 256 else 1.0), 4), "fa_bwd_dq": round(3 * fwd, 4),
            "fa_bwd_dkdv": round(dkdv, 4), "fa_bwd_fused": round(dkdv, 4)}


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed, so
    that an edit of comments alone does not count as a change of the kernel."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_attention_03_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None.

    The summary file (profiles/traffic_<kernel>_<workload>.txt) holds
    key = value lines: fetch_bytes, write_bytes (already scaled by the
    copy-kernel calibration) and source_hash.  A hash that no longer matches
    the kernel's sources means the kernel changed since the counters were
    taken, and the figure is not reported.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    if kv.get("source_hash") != sources_hash(kernel):
        return None
    try:
        return float(kv["fetch_bytes"]) + float(kv["write_bytes"])
    except (KeyError, ValueError):
        return None


def stored_mfma_busy(kernel: str, workload: str):
    """Share of the dispatch's SIMD cycles in which the matrix unit was busy,
    from a committed rocprofv3 counter summary
    (profiles/mfma_<kernel>_<workload>.txt: SQ_VALU_MFMA_BUSY_CYCLES over
    GRBM_GUI_ACTIVE per XCD x CUs x 4), or None when absent or when the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"mfma_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    if kv.get("source_hash") != sources_hash(kernel):
        return None
    try:
        return float(kv["mfma_busy"])
    except (KeyError, ValueError):
        return None


def stored_clock(kernel: str, workload: str):
    """Engine clock (GHz) measured during the kernel, from a committed
    rocprofv3 GRBM summary (profiles/clock_fwd_bwd_<workload>.txt), or None
    when absent or when the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"clock_fwd_bwd_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    if kv.get(f"{kernel}_hash") != sources_hash(kernel):
        return None
    try:
        return float(kv[f"{kernel}_ghz"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ CPU baseline
def _oracle_heads(args):
    """Worker: fp64 oracle forward + backward over a list of (q, k, v, do) problems."""
    import numpy as np

    import oracle

    problems, scale, causal = args
    for q, k, v, do in problems:
        oracle.attention_backward(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                  do.astype(np.float64), scale, causal)
    return len(problems)


def _problems(w, cpu_inputs, n_heads: int):
    """The first n_heads (sequence, query head) problems of the workload as
    float32 (q, k, v, do) arrays, each query head with the key/value head it
    shares (the grouped oracle's per-head work; its sum of dK / dV over a
    group is not timed), and the lengths of their sequences."""
    G = w.H // w.kv_heads
    q, k, v, do = cpu_inputs
    f = lambda t: t.float().numpy()  # noqa: E731  (one problem at a time)
    out, lens = [], []
    if w.varlen:
        cu = w.cu_seqlens
        for b in range(w.Z):
            for h in range(w.H):
                if len(out) == n_heads:
                    return out, lens
                s, e = int(cu[b]), int(cu[b + 1])
                out.append((f(q[h, s:e]), f(k[h // G, s:e]), f(v[h // G, s:e]), f(do[h, s:e])))
                lens.append(e - s)
        return out, lens
    for z in range(w.Z):
        for h in range(w.H):
            if len(out) == n_heads:
                return out, lens
            out.append((f(q[z, h]), f(k[z, h // G]), f(v[z, h // G]), f(do[z, h])))
            lens.append(w.N)
    return out, lens


def cpu_baseline(w, cpu_inputs, n_heads: int, workers: int):
    """Time the oracle (as it stands) over the first n_heads heads of the workload."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np

    problems, lens = _problems(w, cpu_inputs, n_heads)
    workers = max(1, min(workers, len(problems)))
    chunks = np.array_split(np.arange(len(problems)), workers)
    jobs = [([problems[i] for i in c], w.scale, w.causal) for c in chunks if len(c)]
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"  # one BLAS thread per worker process
    try:
        with cf.ProcessPoolExecutor(max_workers=len(jobs), mp_context=mp.get_context("spawn")) as ex:
            list(ex.map(_oracle_heads, [(j[0][:1],) + j[1:] for j in jobs]))  # warm import
            t0 = time.perf_counter()
            done = sum(ex.map(_oracle_heads, jobs))
            dt = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    per = 4.0 * w.D * float(sum(n * n for n in lens[:done])) * (0.5 if w.causal else 1.0)
    flops = 3.5 * per
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": len(jobs),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, fwd+bwd (full N x N S and P, naive backward) on {done} of "
                   f"{w.Z * w.H} (sequence, head) problems of the same seeded workload, {len(jobs)} processes x 1 BLAS "
                   f"thread, wall {dt:.2f} s; FLOPs counted with the same convention"),
    }


# ------------------------------------------------------------------ GPU timing
def run(args, workload=None, steps=None, warmup=None, side=False, bwd=None):
    """One JSON record of the step on a workload (args.workload by default).
    side=True: a secondary configuration of the default run (no CPU baseline,
    no calibration copy, no standalone Delta pass).  bwd: "split" (dQ pass
    with the statistics, then the dK/dV pass) or "fused" (statistics pass,
    then the fused per-head pass); args.bwd by default."""
    import torch

    import exact_attention_03_amd as fa

    w = workloads.by_name(workload or args.workload)
    n_steps = args.steps if steps is None else steps
    n_warm = args.warmup if warmup is None else warmup
    variant = bwd or args.bwd
    kernels = KERNELS_FUSED if variant == "fused" else KERNELS
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cpu_inputs = workloads.make_inputs(w)
    q, k, v, do = (t.to(dev) for t in cpu_inputs)
    Z, H, N, D = w.shape
    Hkv = w.kv_heads
    T = w.T
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stats = torch.empty((2,) + tuple(q.shape[:-1]), dtype=torch.float32, device=dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev) if w.varlen else None
    L = fa.lib()
    code = fa._dtype_code(q)
    causal = int(w.causal)
    scale = w.scale
    P = lambda t: t.data_ptr()  # noqa: E731
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def call(st, name):
        if st != 0:
            raise fa.FAError(st, name, fa.last_error())

    def step_varlen(ev=None):
        if ev is not None:
            ev[0].record(stream)
        call(L.fa_fwd_varlen(Z, H, Hkv, T, N, D, code, code, P(cu), P(q), P(k), P(v), P(o), P(lse), scale, causal,
                             sp), "fa_fwd_varlen")
        if ev is not None:
            ev[1].record(stream)
        call(L.fa_bwd_dq_and_stats_varlen(Z, H, Hkv, T, N, D, code, code, P(cu), P(q), P(k), P(v), P(o), P(do),
                                          P(lse), P(stats), P(dq), scale, causal, sp), "fa_bwd_dq_and_stats_varlen")
        if ev is not None:
            ev[2].record(stream)
        call(L.fa_bwd_dkdv_varlen(Z, H, Hkv, T, N, D, code, P(cu), P(q), P(k), P(v), P(do), P(stats), P(dk), P(dv),
                                  scale, causal, 0, sp), "fa_bwd_dkdv_varlen")
        if ev is not None:
            ev[3].record(stream)

    part = None
    if variant == "fused":
        if w.varlen or Hkv != H:
            raise SystemExit("bench.py: the fused backward takes plain heads and dense batches only")
        part = torch.empty((L.fa_bwd_fused_workspace_bytes(Z, H, N, D) // 4,), dtype=torch.float32, device=dev)

    def step_fused(ev=None):
        if ev is not None:
            ev[0].record(stream)
        call(L.fa_fwd(Z, H, N, D, code, code, P(q), P(k), P(v), P(o), P(lse), scale, causal, sp), "fa_fwd")
        if ev is not None:
            ev[1].record(stream)
        call(L.fa_bwd_preprocess(Z, H, N, D, code, code, P(o), P(do), P(lse), P(stats), sp), "fa_bwd_preprocess")
        if ev is not None:
            ev[2].record(stream)
        call(L.fa_bwd_fused(Z, H, N, D, code, P(q), P(k), P(v), P(do), P(stats), P(dq), P(dk), P(dv), scale, causal,
                            0, P(part), part.numel() * 4, sp), "fa_bwd_fused")
        if ev is not None:
            ev[3].record(stream)

    def step(ev=None):
        # Grouped key/value heads go through the *_gqa forms of the same calls,
        # variable-length batches through the *_varlen forms.
        if variant == "fused":
            return step_fused(ev)
        if w.varlen:
            return step_varlen(ev)
        if ev is not None:
            ev[0].record(stream)
        if Hkv == H:
            call(L.fa_fwd(Z, H, N, D, code, code, P(q), P(k), P(v), P(o), P(lse), scale, causal, sp), "fa_fwd")
        else:
            call(L.fa_fwd_gqa(Z, H, Hkv, N, D, code, code, P(q), P(k), P(v), P(o), P(lse), scale, causal, sp),
                 "fa_fwd_gqa")
        if ev is not None:
            ev[1].record(stream)
        if Hkv == H:
            call(L.fa_bwd_dq_and_stats(Z, H, N, D, code, code, P(q), P(k), P(v), P(o), P(do), P(lse), P(stats),
                                       P(dq), scale, causal, sp), "fa_bwd_dq_and_stats")
        else:
            call(L.fa_bwd_dq_and_stats_gqa(Z, H, Hkv, N, D, code, code, P(q), P(k), P(v), P(o), P(do), P(lse),
                                           P(stats), P(dq), scale, causal, sp), "fa_bwd_dq_and_stats_gqa")
        if ev is not None:
            ev[2].record(stream)
        if Hkv == H:
            call(L.fa_bwd_dkdv(Z, H, N, D, code, P(q), P(k), P(v), P(do), P(stats), P(dk), P(dv),
                               scale, causal, 0, sp), "fa_bwd_dkdv")
        else:
            call(L.fa_bwd_dkdv_gqa(Z, H, Hkv, N, D, code, P(q), P(k), P(v), P(do), P(stats), P(dk), P(dv),
                                   scale, causal, 0, sp), "fa_bwd_dkdv_gqa")
        if ev is not None:
            ev[3].record(stream)

    if args.calib_copy_mib > 0 and not side:
        # A plain device copy of known size, for scaling HBM counters.
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(n_warm):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(n_steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(n_steps):
        step(evs[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / n_steps
    per = {name: [] for name in kernels}
    for e in evs:
        for i, name in enumerate(kernels):
            per[name].append(e[i].elapsed_time(e[i + 1]))
    avg = {n: sum(x) / len(x) for n, x in per.items()}
    step_times = sorted(e[0].elapsed_time(e[-1]) for e in evs)  # first launch to last completion
    spread = {"median": round(step_times[len(step_times) // 2], 4), "min": round(step_times[0], 4),
              "max": round(step_times[-1], 4)}

    # The standalone Delta pass (fa_bwd_preprocess), outside the step (the
    # step's dQ pass computes the same statistics): its HBM rate.
    delta = None
    if not w.varlen and Hkv == H and not side:
        stats2 = torch.empty_like(stats)
        pre = lambda: call(L.fa_bwd_preprocess(Z, H, N, D, code, code, P(o), P(do), P(lse), P(stats2), sp),  # noqa
                           "fa_bwd_preprocess")
        for _ in range(3):
            pre()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(20):
            pre()
        e1.record(stream)
        torch.cuda.synchronize()
        pre_ms = e0.elapsed_time(e1) / 20
        pre_bytes = kernel_work(w, o.element_size())["fa_bwd_pre"][1]
        delta = {"ms": round(pre_ms, 4), "GB/s": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1),
                 "frac": round(pre_bytes / (pre_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bytes": pre_bytes,
                 "traffic": stored_traffic("fa_bwd_pre", w.name), "in_step": False}

    ff = fwd_flops(w)
    fwd_ms = avg["fa_fwd"]
    bwd_ms = sum(avg[n] for n in kernels[1:])
    value = 3.5 * ff / (ms_step * 1e-3) / 1e12
    work = kernel_work(w, o.element_size())
    ratio = executed_over_counted(w)
    n_cu = fa.device_info(D)[0]
    kern = {}
    for name in kernels:
        bound, amount, unit = work[name]
        t = avg[name] * 1e-3
        if bound == "mfma":
            ach = amount / t / 1e12
            kern[name] = {"ms": round(avg[name], 4), "bound": "mfma", "TFLOP/s": round(ach, 1),
                          "frac": round(ach / PEAK_MFMA_F16_TFLOPS, 4), "executed_over_counted": ratio[name],
                          "executed_TFLOP/s": round(ach * ratio[name], 1)}
            busy = stored_mfma_busy(name, w.name)
            if busy is not None:
                kern[name]["mfma_busy"] = busy
            clk = stored_clock(name, w.name)
            if clk is not None:
                # the dense fp16 rate at the clock the kernel actually ran at: CUs x clock x 4096
                peak_clk = n_cu * clk * 4096 / 1e3
                kern[name].update({"observed_clock_GHz": clk, "peak_at_observed_clock_TFLOP/s": round(peak_clk, 1),
                                   "frac_at_observed_clock": round(ach / peak_clk, 4)})
        else:
            ach = amount / t / 1e9
            kern[name] = {"ms": round(avg[name], 4), "bound": "hbm", "GB/s": round(ach, 1),
                          "frac": round(ach / PEAK_HBM_GBS, 4)}
    dom = max(kernels, key=lambda n: avg[n])
    bound, amount, unit = work[dom]
    t = avg[dom] * 1e-3
    traffic = stored_traffic(dom, w.name)
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(amount / t / 1e12, 1), "peak": PEAK_MFMA_F16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(amount / t / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["algorithmic"] = {"amount": amount, "unit": unit, "per_launch": True}

    out = {
        "metric": "FlashAttention fwd+bwd TFLOP/s on 1 MI355X, % of fp16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": n_warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: " + (f"B={Z} sequences of {min(w.lengths)}..{N} tokens (T={T}) "
                                                 if w.varlen else f"Z={Z} ") + f"H={H}" +
                               (f" Hkv={Hkv}" if Hkv != H else "") + ("" if w.varlen else f" N={N}") +
                               f" D={D} {w.dtype} causal={bool(w.causal)} scale={scale:.9g}",
                   "Z": Z, "H": H, "Hkv": Hkv, "N": N, "D": D, "causal": bool(w.causal), "seed": w.seed},
        "frac_of_peak": round(value / PEAK_MFMA_F16_TFLOPS, 4),
        "breakdown": {
            "bwd_variant": variant,
            "step_ms": spread,
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_TFLOP/s": round(ff / (fwd_ms * 1e-3) / 1e12, 1),
            "bwd_TFLOP/s": round(2.5 * ff / (bwd_ms * 1e-3) / 1e12, 1),
            "fwd_frac": round(ff / (fwd_ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
            "bwd_frac": round(2.5 * ff / (bwd_ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
            "kernels": kern,
            "delta_pass": delta,
        },
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and not side:
        out["cpu_baseline"] = cpu_baseline(w, cpu_inputs, args.cpu_heads, args.cpu_workers)
    return out


SIDE_CONFIGS = ("d64", "d256_bf16", "long_causal_bf16")
AB_CONFIGS = ("d128_causal", "long_causal_bf16")


def backward_ab(args, main) -> dict:
    """The whole backward both ways on the A/B workloads: the two-pass form
    (dQ pass with the statistics, then dK/dV) against the fused per-head form
    (statistics pass, then dQ/dK/dV in one pass), at most 20 timed steps
    each; the main line's own variant is taken from it."""
    import torch

    res = {}
    for name in AB_CONFIGS:
        row = {}
        for variant in ("split", "fused"):
            if name == main["config"]["workload"].split(":")[0] and variant == main["breakdown"]["bwd_variant"]:
                r = main
            else:
                r = run(args, workload=name, steps=min(args.steps, 20), warmup=min(args.warmup, 5), side=True,
                        bwd=variant)
            b = r["breakdown"]
            row[variant] = {"bwd_ms": b["bwd_ms"], "bwd_TFLOP/s": b["bwd_TFLOP/s"], "bwd_frac": b["bwd_frac"],
                            "kernels_ms": {n: k["ms"] for n, k in b["kernels"].items() if n != "fa_fwd"}}
            torch.cuda.empty_cache()
        row["faster"] = min(("split", "fused"), key=lambda v: row[v]["bwd_ms"])
        res[name] = row
        print(f"bench: backward A/B {name}: split {row['split']['bwd_ms']} ms, fused {row['fused']['bwd_ms']} ms",
              file=sys.stderr, flush=True)
    return res


def side_configs(args) -> dict:
    """fwd, bwd and fwd+bwd throughput of the other full-size workloads (the
    same step, at most 20 timed steps each), for the default run's line."""
    import torch

    res = {}
    for name in SIDE_CONFIGS:
        r = run(args, workload=name, steps=min(args.steps, 20), warmup=min(args.warmup, 5), side=True)
        b = r["breakdown"]
        res[name] = {"workload": r["config"]["workload"], "steps": r["steps"], "ms_per_step": r["ms_per_step"],
                     "fwd_ms": b["fwd_ms"], "bwd_ms": b["bwd_ms"],
                     "fwd_TFLOP/s": b["fwd_TFLOP/s"], "bwd_TFLOP/s": b["bwd_TFLOP/s"],
                     "fwd_bwd_TFLOP/s": r["value"], "fwd_frac": b["fwd_frac"], "bwd_frac": b["bwd_frac"],
                     "fwd_bwd_frac": r["frac_of_peak"],
                     "kernels_ms": {n: k["ms"] for n, k in b["kernels"].items()}}
        print(f"bench: {name} {r['value']} TFLOP/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ paged decode
def decode_bytes(w, lens) -> float:
    """Algorithmic HBM bytes of one decode step: the new tokens' K / V rows
    read and written into the cache (q_len per sequence), every cached K and
    V element of the contexts read once, q read, O (16-bit) and lse written
    (q_len rows per sequence), the block-table entries of the contexts, the
    context lengths and (q_len > 1) the per-row visible lengths read."""
    import numpy as np

    lens = np.asarray(lens, dtype=np.int64)
    e = 2  # bytes per 16-bit element
    n = len(lens)
    T = w.q_len
    ctx = float(lens.sum()) * w.Hkv * w.D * 2 * e
    new = float(n) * T * w.Hkv * w.D * 2 * e * 2
    qo = float(n) * T * (w.H * w.D * e * 2 + w.H * 4)
    tables = float((-(-lens // w.block_size)).sum()) * 4 + n * 4 + (n * T * 4 if T > 1 else 0)
    return ctx + new + qo + tables


def _oracle_decode(args):
    import oracle

    q, kc, vc, tables, lens, scale, topk, win = args
    if q.ndim == 4:  # several query tokens per sequence: the last ones of each context, each causal
        T = q.shape[1]
        rows = [[int(n) - T + t + 1 for t in range(T)] for n in lens]
        src = {"k_cache": kc, "v_cache": vc, "block_tables": tables, "context_lens": lens, "row_lens": rows}
        oracle.attention_over_sources(q, [src], scale)
        return len(lens)
    if not topk:
        oracle.paged_decode(q, kc, vc, tables, lens, scale)
        return len(lens)
    # query-aware: page min / max, scores, Top-K, attention over the kept pages
    n_kv = kc.shape[1]
    G = q.shape[1] // n_kv
    selected = []
    for b in range(len(lens)):
        row = []
        for hk in range(n_kv):
            mn, mx = oracle.quest_page_minmax(kc, tables[b], int(lens[b]), hk)
            row.append(oracle.quest_select(oracle.quest_scores(q[b, hk * G:(hk + 1) * G], mn, mx), topk))
        selected.append(row)
    if win is None:
        oracle.quest_sparse_decode(q, kc, vc, tables, lens, selected, scale)
    else:  # the window pool and the kept pages under one softmax
        pool = {"k_cache": kc, "v_cache": vc, "block_tables": tables, "context_lens": lens, "selected": selected}
        window = {"k_cache": win[0], "v_cache": win[1], "block_tables": win[2], "context_lens": win[3]}
        oracle.decode_over_sources(q, [window, pool], scale)
    return len(lens)


def _subset_pages(cache, c):
    """The pages of sequences c of a (q, k_cache, v_cache, tables, lens)
    cache, renumbered: (k_cache, v_cache, tables, lens) as float32 / int32."""
    import numpy as np

    _, kc, vc, tables, lens = cache
    t = tables[c].numpy()
    used = sorted({int(x) for x in t.flatten() if x >= 0})
    remap = {b: i for i, b in enumerate(used)}
    t2 = np.vectorize(lambda x: remap.get(int(x), -1))(t).astype(np.int32)
    return kc[used].float().numpy(), vc[used].float().numpy(), t2, lens[c].numpy()


def decode_cpu_baseline(w, cpu, n_seq: int, workers: int, window=None):
    """The paged-decode oracle on the first n_seq sequences (one process per
    chunk of sequences, one BLAS thread each), in the same GB/s unit; with a
    window pool (its inputs), the two-source oracle."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np

    q, kc, vc, tables, lens = cpu
    n_seq = min(n_seq, w.B)
    # The oracle reads only the pages of the sampled sequences: hand each
    # worker those pages, renumbered.
    jobs = []
    for c in np.array_split(np.arange(n_seq), max(1, min(workers, n_seq))):
        if not len(c):
            continue
        jobs.append((q[c].float().numpy(), *_subset_pages(cpu, c), w.scale, w.topk,
                     _subset_pages(window, c) if window is not None else None))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        with cf.ProcessPoolExecutor(max_workers=len(jobs), mp_context=mp.get_context("spawn")) as ex:
            t0 = time.perf_counter()
            done = sum(ex.map(_oracle_decode, jobs))
            dt = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    sub = lens[:done].numpy()
    nbytes = sum(quest_bytes(w, sub)) if w.topk else decode_bytes(w, sub)
    what = ("query-aware oracle (page min / max, scores, Top-K, attention over the kept pages)" if w.topk
            else "paged-decode oracle (token-by-token gather through the block table, plain softmax)")
    if w.q_len > 1:
        what = f"paged oracle with {w.q_len} causal query rows per sequence (per-row visible lengths)"
    if window is not None:
        what = ("query-aware oracle (page min / max, scores, Top-K) and the two-source oracle (window pool and kept "
                "pages under one softmax)")
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": len(jobs), "kind": "oracle",
            "sample": (f"fp64 numpy {what} on {done} of {w.B} sequences ({int(sub.sum())} context tokens) of the "
                       f"same seeded workload, {len(jobs)} processes x 1 BLAS thread, wall {dt:.2f} s (process "
                       f"start included); bytes counted as for the GPU")}


def quest_bytes(w, lens):
    """Algorithmic HBM bytes of one query-aware step: the selection reads q,
    the block-table entries and the min / max of every page of each context
    and writes the kept page lists; the sparse decode reads the kept pages'
    valid K and V tokens, q, the lists and the table entries of the kept pages,
    and writes O (16-bit) and lse; with a window pool it also reads the
    window's K and V tokens and table entries.  Returns (selection bytes,
    decode bytes)."""
    import numpy as np

    lens = np.asarray(lens, dtype=np.int64)
    e = 2
    pages = -(-lens // w.block_size)
    sel = (float(pages.sum()) * w.Hkv * 2 * w.D * e + float(pages.sum()) * 4 + w.B * w.H * w.D * e
           + w.B * w.Hkv * (w.topk + 1) * 4)
    kept_tokens = 0.0
    for n, p in zip(lens, pages):
        k = min(int(p), w.topk)
        # the kept pages are full except possibly the context's last page
        kept_tokens += k * w.block_size - (w.block_size * p - n if k == p else 0)
    dec = (kept_tokens * w.Hkv * w.D * 2 * e + w.B * w.H * w.D * e * 2 + w.B * w.H * 4
           + w.B * w.Hkv * (w.topk + 1) * 4 + float(np.minimum(pages, w.topk).sum()) * w.Hkv * 4)
    if w.window:
        wpages = -(-w.window // w.block_size)
        dec += len(lens) * (float(w.window) * w.Hkv * w.D * 2 * e + wpages * w.Hkv * 4)
    return sel, dec


def run_quest(args):
    """One step = fa_quest_select (scores of every page, Top-K) + fa_paged_decode_sparse
    over the kept pages.  The page min / max are computed once before timing (a
    serving engine updates them as pages fill)."""
    import numpy as np
    import torch

    import exact_attention_03_amd as fa

    from exact_attention_03_amd._lib import KvSource

    w = workloads.DECODE_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cpu = workloads.make_decode_inputs(w)
    q, kc, vc, tables, lens = (t.to(dev) for t in cpu)
    lens_np = cpu[4].numpy().astype(np.int64)
    kmeta = fa.quest_page_minmax(kc, tables, lens)
    wcpu = workloads.make_decode_inputs(w.window_pool()) if w.window else None
    sel = torch.empty((w.B, w.Hkv, w.topk), dtype=torch.int32, device=dev)
    nsel = torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev)
    o = torch.empty((w.B, w.H, w.D), dtype=q.dtype, device=dev)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    L = fa.lib()
    code = fa._dtype_code(q)
    nb, mxb = kc.shape[0], tables.shape[1]
    P = lambda t: t.data_ptr()  # noqa: E731
    if w.window:
        # source 0: the window pool attended whole; source 1: the kept pages
        _, wkc, wvc, wtab, wlens = (t.to(dev) for t in wcpu)
        srcs = (KvSource * 2)(
            KvSource(P(wkc), P(wvc), P(wtab), P(wlens), w.block_size, wkc.shape[0], wtab.shape[1], w.window,
                     None, None, 0),
            KvSource(P(kc), P(vc), P(tables), P(lens), w.block_size, nb, mxb, 0, P(sel), P(nsel), w.topk))
        ws_bytes = L.fa_paged_decode_sources_workspace_bytes(w.B, w.H, w.Hkv, w.D, 2, srcs)
    else:
        ws_bytes = L.fa_paged_decode_workspace_bytes(w.B, w.H, w.Hkv, w.D, w.topk * w.block_size)
    ws = torch.empty((max(1, ws_bytes // 4),), dtype=torch.float32, device=dev)
    dec_name = "fa_paged_decode_sources" if w.window else "fa_paged_decode_sparse"
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def call(st, name):
        if st != 0:
            raise fa.FAError(st, name, fa.last_error())

    if args.calib_copy_mib > 0:
        # A plain device copy of known size, for scaling HBM counters.
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        call(L.fa_quest_select(w.B, w.H, w.Hkv, w.D, w.block_size, nb, mxb, w.topk, code, P(q), P(kmeta), P(tables),
                               P(lens), P(sel), P(nsel), sp), "fa_quest_select")
        if ev is not None:
            ev[1].record(stream)
        if w.window:
            call(L.fa_paged_decode_sources(w.B, w.H, w.Hkv, w.D, code, code, P(q), 2, srcs, P(o), P(lse), w.scale,
                                           P(ws), ws_bytes, sp), dec_name)
        else:
            call(L.fa_paged_decode_sparse(w.B, w.H, w.Hkv, w.D, w.block_size, nb, mxb, w.topk, code, code, P(q),
                                          P(kc), P(vc), P(tables), P(lens), P(sel), P(nsel), P(o), P(lse), w.scale,
                                          P(ws), ws_bytes, sp), dec_name)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    sel_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    sel_b, dec_b = quest_bytes(w, lens_np)
    kern = {"fa_quest_select": (sel_ms, sel_b), dec_name: (dec_ms, dec_b)}
    dom = max(kern, key=lambda k: kern[k][0])
    ach = kern[dom][1] / (kern[dom][0] * 1e-3) / 1e9
    metric = ("query-aware sparse decode (page selection + attention over the kept pages) HBM GB/s on 1 MI355X"
              if not w.window else
              "two-source sparse decode (page selection + attention over a sliding-window pool and the kept pages "
              "under one softmax) HBM GB/s on 1 MI355X")
    window_txt = f", plus a window pool of {w.window} tokens per sequence" if w.window else ""
    out = {
        "metric": metric,
        "value": round((sel_b + dec_b) / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} sequences, contexts {int(lens_np.min())}..{int(lens_np.max())} "
                               f"tokens, H={w.H} Hkv={w.Hkv} D={w.D} pages of {w.block_size} tokens, {w.topk} pages "
                               f"kept per context{window_txt}, {w.dtype}",
                   "B": w.B, "H": w.H, "Hkv": w.Hkv, "D": w.D, "block_size": w.block_size, "topk": w.topk,
                   "window": w.window, "seed": w.seed},
        "breakdown": {"select_ms": round(sel_ms, 4), "sparse_decode_ms": round(dec_ms, 4),
                      "select_GB/s": round(sel_b / (sel_ms * 1e-3) / 1e9, 1),
                      "sparse_decode_GB/s": round(dec_b / (dec_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": stored_traffic(dom, w.name) if dom in KERNEL_SOURCES else None, "kernel": dom,
                     "algorithmic": {"amount": kern[dom][1], "unit": "byte", "per_launch": True}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = decode_cpu_baseline(w, cpu, args.cpu_decode_seqs, args.cpu_workers, wcpu)
    return out


def run_decode(args):
    """One step = fa_reshape_and_cache of the new tokens (the last q_len
    positions of each context) + attention of those tokens over the whole
    context: fa_paged_decode for one token, fa_paged_attention_sources with
    per-row visible lengths (each token causal) for several."""
    import numpy as np
    import torch

    import exact_attention_03_amd as fa
    from exact_attention_03_amd._lib import KvSource

    w = workloads.DECODE_WORKLOADS[args.workload]
    T = w.q_len
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cpu = workloads.make_decode_inputs(w)
    q, kc, vc, tables, lens = (t.to(dev) for t in cpu)
    lens_np = cpu[4].numpy().astype(np.int64)
    tab_np = cpu[3].numpy()
    pos = [(b, int(n) - T + t) for b, n in enumerate(lens_np) for t in range(T)]
    slots = torch.tensor([int(tab_np[b, p // w.block_size]) * w.block_size + p % w.block_size for b, p in pos],
                         dtype=torch.int64, device=dev)
    gen = torch.Generator().manual_seed(w.seed)
    new_k = torch.randn((w.B * T, w.Hkv, w.D), generator=gen).to(q.dtype).to(dev)
    new_v = torch.randn((w.B * T, w.Hkv, w.D), generator=gen).to(q.dtype).to(dev)
    o = torch.empty(tuple(q.shape), dtype=q.dtype, device=dev)
    lse = torch.empty(tuple(q.shape[:-1]), dtype=torch.float32, device=dev)
    L = fa.lib()
    code = fa._dtype_code(q)
    nb, mxb = kc.shape[0], tables.shape[1]
    P = lambda t: t.data_ptr()  # noqa: E731
    if T > 1:
        rows = torch.tensor([[int(n) - T + t + 1 for t in range(T)] for n in lens_np], dtype=torch.int32, device=dev)
        srcs = (KvSource * 1)(KvSource(P(kc), P(vc), P(tables), P(lens), w.block_size, nb, mxb, w.hi, None, None, 0,
                                       P(rows)))
        ws_bytes = L.fa_paged_attention_sources_workspace_bytes(w.B, T, w.H, w.Hkv, w.D, 1, srcs)
        dec_name = "fa_paged_attention_sources"
    else:
        ws_bytes = L.fa_paged_decode_workspace_bytes(w.B, w.H, w.Hkv, w.D, w.hi)
        dec_name = "fa_paged_decode"
    ws = torch.empty((max(1, ws_bytes // 4),), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def call(st, name):
        if st != 0:
            raise fa.FAError(st, name, fa.last_error())

    if args.calib_copy_mib > 0:
        # A plain device copy of known size, for scaling HBM counters.
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        call(L.fa_reshape_and_cache(w.B * T, w.Hkv, w.D, w.block_size, nb, code, P(new_k), P(new_v), P(slots),
                                    P(kc), P(vc), sp), "fa_reshape_and_cache")
        if ev is not None:
            ev[1].record(stream)
        if T > 1:
            call(L.fa_paged_attention_sources(w.B, T, w.H, w.Hkv, w.D, code, code, P(q), 1, srcs, P(o), P(lse),
                                              w.scale, P(ws), ws_bytes, sp), dec_name)
        else:
            call(L.fa_paged_decode(w.B, w.H, w.Hkv, w.D, w.block_size, nb, mxb, w.hi, code, code, P(q), P(kc),
                                   P(vc), P(tables), P(lens), P(o), P(lse), w.scale, P(ws), ws_bytes, sp), dec_name)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    cache_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    nbytes = decode_bytes(w, lens_np)
    dec_bytes = nbytes - float(w.B) * T * w.Hkv * w.D * 2 * 2 * 2  # the cache write's bytes are the other kernel's
    splits = max(1, ws_bytes // (4 * w.B * T * w.H * (w.D + 1))) if ws_bytes else 1
    ach = dec_bytes / (dec_ms * 1e-3) / 1e9
    metric = ("paged decode attention (cache write + decode) HBM GB/s on 1 MI355X" if T == 1 else
              f"causal chunk over a paged cache (cache write of {T} tokens + attention of {T} causal "
              f"query tokens per sequence) HBM GB/s on 1 MI355X")
    out = {
        "metric": metric,
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} sequences, contexts {int(lens_np.min())}..{int(lens_np.max())} "
                               f"tokens ({int(lens_np.sum())} total), H={w.H} Hkv={w.Hkv} D={w.D} pages of "
                               f"{w.block_size} tokens, {w.dtype}, {splits} context splits"
                               + (f", {T} query tokens per sequence" if T > 1 else ""),
                   "B": w.B, "H": w.H, "Hkv": w.Hkv, "D": w.D, "block_size": w.block_size, "q_len": T,
                   "seed": w.seed},
        "breakdown": {"reshape_and_cache_ms": round(cache_ms, 4), "paged_decode_ms": round(dec_ms, 4),
                      "splits": splits},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": stored_traffic(dec_name, w.name),
                     "kernel": f"{dec_name} (decode kernel and, with splits, its combine kernel)",
                     "algorithmic": {"amount": dec_bytes, "unit": "byte", "per_launch": True}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = decode_cpu_baseline(w, cpu, args.cpu_decode_seqs, args.cpu_workers)
    return out


def device_record() -> dict:
    """What the numbers were measured on: device name and CU count, ROCm/HIP,
    torch and numpy versions."""
    import numpy as np
    import torch

    import exact_attention_03_amd as fa

    return {"name": torch.cuda.get_device_name(0), "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", ""),
            "compute_units": fa.device_info(128)[0], "hip": torch.version.hip, "torch": torch.__version__,
            "numpy": np.__version__}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(workloads.WORKLOADS) + sorted(workloads.DECODE_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-heads", type=int, default=1024, help="heads in the oracle timing sample")
    ap.add_argument("--bwd", choices=("split", "fused"), default="split",
                    help="backward form of the step: dQ pass + dK/dV pass, or statistics + fused per-head pass")
    ap.add_argument("--no-configs", action="store_true",
                    help="default workload only: skip the other full-size workloads in the 'configs' object")
    ap.add_argument("--cpu-workers", type=int, default=min(16, len(os.sched_getaffinity(0))))
    ap.add_argument("--cpu-decode-seqs", type=int, default=64, help="sequences in the decode oracle timing sample")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before warm-up, copy a buffer of this many MiB (for HBM counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested). Attention heads are "
              "independent, so a multi-GPU run would shard Z*H across GPUs with no exchange; it is not "
              "implemented here.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")
    if args.workload in workloads.DECODE_WORKLOADS:
        out = run_quest(args) if workloads.DECODE_WORKLOADS[args.workload].topk else run_decode(args)
    else:
        out = run(args)
        if args.workload == DEFAULT_WORKLOAD and not args.no_configs:
            out["configs"] = side_configs(args)
            out["bwd_ab"] = backward_ab(args, out)
    out["device"] = device_record()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
