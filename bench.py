#!/usr/bin/env python3
"""Fused MHA forward benchmark on one MI355X.

One step = one call of the fused forward (the whole hot path is one kernel launch)
over the workload's inputs, already resident in HBM.  Prints ONE JSON line:
TFLOP/s credited as 4*B*H*N^2*d (halved for causal) per second, the roofline of the
kernel (MFMA-bound; achieved TFLOP/s from HIP events over the timed region on the
launch stream, against the published dense bf16 peak), and the CPU oracle timed on a
bounded sample of the same workload on the host cores.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--sweep]
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
sys.path.insert(0, ROOT)

METRIC = "fused MHA fwd TFLOP/s + % of bf16 MFMA peak (B4 H32 N4096 d128 causal)"
HEADLINE = "bf16_B4_H32_N4096_d128_causal"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X published dense peaks
HBM_GBS = 8000.0


KERNEL_SOURCES = ("mha_fwd_kernel.hip", "mha_layout.h", "gfx950_lds.h")


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "head_attention_fa2_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_counters(workload: str) -> dict:
    """Counter figures of the kernel on `workload` taken with rocprofv3 and stored in
    profiles/kernel_counters.json, keyed by the SHA-256 of the kernel sources they were
    taken on; a figure taken on other sources is reported as None.

    traffic_bytes: HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, each scaled by the
    same counter's reading for a plain copy of known size).
    mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x CUs x GRBM_GUI_ACTIVE), the share of
    the launch's cycles in which the matrix cores were busy.
    hbm_gbs: traffic_bytes over the kernel-trace average duration."""
    path = os.path.join(ROOT, "profiles", "kernel_counters.json")
    out = {"traffic_bytes": None, "mfma_busy": None, "hbm_gbs": None}
    try:
        with open(path, encoding="utf-8") as fh:
            entry = json.load(fh).get(workload)
    except (OSError, ValueError):
        return out
    if not entry or entry.get("kernel_source_sha256") != kernel_source_sha256():
        return out
    for key in out:
        out[key] = entry.get(key)
    return out


def _to_device(a, dtype, dev):
    import numpy as np
    import torch

    if dtype in ("bf16", "f16"):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def time_gpu(w, steps, warmup, dev, settle_s=0.0):
    """Settle the clock, warm up, then time exactly `steps` launches bracketed by
    synchronisations, with a HIP event on the launch stream between launches."""
    import torch

    import head_attention_fa2_amd as mha
    import mha_inputs

    q, k, v = mha_inputs.draw_qkv(w)
    tq, tk, tv = (_to_device(x, w.dtype, dev) for x in (q, k, v))
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        mha.fwd(tq, tk, tv, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)

    settle = settle_clock(call, dev, settle_s)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]      # ms, per launch
    total_ms = ev[0].elapsed_time(ev[steps])
    return dict(total_ms=total_ms, per_ms=per, wall_s=wall, settle=settle, inputs=(q, k, v), out=(o, lse))


def time_vs_torch(w, passes, reps, dev):
    """This library's forward and torch's fused attention (its flash backend only, so that
    torch never takes its unfused math path) on the same device inputs, timed in
    alternating passes after a clock settle; medians of the passes, in ms per launch.
    None when torch has no flash kernel for the shape or element type."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    import head_attention_fa2_amd as mha
    import mha_inputs

    q, k, v = mha_inputs.draw_qkv(w)
    tq, tk, tv = (_to_device(x, w.dtype, dev) for x in (q, k, v))
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def ours():
        mha.fwd(tq, tk, tv, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)

    def theirs():
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            return F.scaled_dot_product_attention(tq, tk, tv, is_causal=w.causal, scale=w.scale)

    try:
        ref = theirs()
        torch.cuda.synchronize(dev)
    except (RuntimeError, NotImplementedError, ValueError) as e:   # no flash kernel for this case
        return {"torch_flash": None, "reason": (str(e).splitlines() or [type(e).__name__])[0][:160]}
    settle_clock(lambda: (ours(), theirs()), dev, 1.0)
    res = {"ours": [], "torch": []}
    for _ in range(passes):
        for key, f in (("ours", ours), ("torch", theirs)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                f()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            res[key].append(e0.elapsed_time(e1) / reps)
    ours()
    torch.cuda.synchronize(dev)
    diff = float((o.float() - ref.float()).abs().max())
    med = {key: sorted(x)[len(x) // 2] for key, x in res.items()}
    return {"ms": med["ours"], "torch_flash_ms": med["torch"], "max_abs_diff_O": diff}


def settle_clock(call, dev, seconds):
    """Launch `call` back to back until `seconds` of wall time have passed (at least one
    launch), synchronising every few launches.  Under sustained load the MI355X lowers
    its clock to its power limit within about a second; timing before that measures a
    clock the workload does not keep.  Returns what ran: seconds and launches."""
    import torch

    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(8):
            call()
        n += 8
        torch.cuda.synchronize(dev)
        el = time.perf_counter() - t0
        if el >= seconds:
            return {"settle_s": round(el, 3), "settle_launches": n}


def time_gpu_splitkv(w, steps, warmup, dev):
    """As time_gpu, for the split-KV forward of a decode workload (library's split count)."""
    import torch

    import head_attention_fa2_amd as mha
    import mha_inputs

    q, k, v = mha_inputs.draw_qkv(w)
    tq, tk, tv = (_to_device(x, w.dtype, dev) for x in (q, k, v))
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(mha.mha_fwd_splitkv_workspace_size(w.B, w.H, w.N, w.Nk, w.d, 0), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        mha.fwd_splitkv(tq, tk, tv, scale=w.scale, out=o, lse=lse, workspace=ws, stream=stream)
    torch.cuda.synchronize(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        mha.fwd_splitkv(tq, tk, tv, scale=w.scale, out=o, lse=lse, workspace=ws, stream=stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    return dict(total_ms=ev[0].elapsed_time(ev[steps]), inputs=(q, k, v), out=(o, lse))


def time_gpu_paged(w, steps, warmup, dev, splits=0):
    """As time_gpu, for the paged split-KV forward of a paged workload."""
    import torch

    import head_attention_fa2_amd as mha
    import mha_inputs

    q, kp, vp, table, lens = mha_inputs.draw_paged_workload(w)
    tq, tk, tv = (_to_device(x, w.dtype, dev) for x in (q, kp, vp))
    tt, tl = torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev)
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(mha.mha_fwd_paged_workspace_size(w.B, w.H, w.Nq, w.d, w.block_size, table.shape[1], splits),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        mha.fwd_paged(tq, tk, tv, tt, tl, scale=w.scale, splits=splits, out=o, lse=lse, workspace=ws, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    return dict(total_ms=ev[0].elapsed_time(ev[1]), inputs=(q, kp, vp, table, lens), out=(o, lse))


def time_gemm(w, steps, warmup, dev, torch_too=True):
    """Time mha.gemm (and torch.matmul, the vendor library, for context) on a GEMM workload."""
    import torch

    import head_attention_fa2_amd as mha
    import mha_inputs

    a, b = mha_inputs.draw_gemm(w.M, w.N, w.K, w.dtype, w.seed)
    ta, tb = _to_device(a, w.dtype, dev), _to_device(b, w.dtype, dev)
    c = torch.empty((w.M, w.N), dtype=ta.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize(dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize(dev)
        return ev[0].elapsed_time(ev[1]) / steps

    # three alternating passes, median of each, so that neither side times on colder clocks
    ours, theirs = [], []
    for _ in range(3):
        ours.append(timed(lambda: mha.gemm(ta, tb, out=c, stream=stream)))
        if torch_too:
            theirs.append(timed(lambda: torch.matmul(ta, tb, out=c)))
    ms = sorted(ours)[1]
    ms_torch = sorted(theirs)[1] if torch_too else None
    mha.gemm(ta, tb, out=c, stream=stream)
    torch.cuda.synchronize(dev)
    return dict(ms=ms, ms_torch=ms_torch, inputs=(a, b), out=c)


def time_gemm_splitk(w, steps, warmup, dev):
    """Time mha.gemm_splitk (library split count) and torch.matmul on a memory-bound GEMM."""
    import torch

    import head_attention_fa2_amd as mha
    import mha_inputs

    a, b = mha_inputs.draw_gemm(w.M, w.N, w.K, w.dtype, w.seed)
    ta, tb = _to_device(a, w.dtype, dev), _to_device(b, w.dtype, dev)
    c = torch.empty((w.M, w.N), dtype=ta.dtype, device=dev)
    ws = torch.empty(mha.mha_gemm_splitk_workspace_size(w.M, w.N, w.K, 0), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize(dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize(dev)
        return ev[0].elapsed_time(ev[1]) / steps

    ms_plain = timed(lambda: mha.gemm(ta, tb, out=c, stream=stream))
    ms_torch = timed(lambda: torch.matmul(ta, tb, out=c))
    ms = timed(lambda: mha.gemm_splitk(ta, tb, out=c, workspace=ws, stream=stream))
    torch.cuda.synchronize(dev)
    return dict(ms=ms, ms_plain=ms_plain, ms_torch=ms_torch, inputs=(a, b), out=c)


def parity_sample_gemm(w, inputs, out, n=8):
    """Largest error / bound over sampled entries of C (<= 1 passes)."""
    import numpy as np
    import torch

    import oracle

    a_bits, b_bits = inputs
    rng = np.random.default_rng(w.seed + 1)
    rows, cols = rng.integers(0, w.M, n), rng.integers(0, w.N, n)
    cg = out[torch.from_numpy(rows).to(out.device)][:, torch.from_numpy(cols).to(out.device)]
    cg = cg.float().cpu().numpy().astype(np.float64)
    a, b = oracle.decode(a_bits[rows], w.dtype), oracle.decode(b_bits[:, cols], w.dtype)
    ratio = np.abs(cg - oracle.gemm(a, b)) / oracle.gemm_error_bound(a, b, w.dtype)
    return {"max_err_over_bound": float(ratio.max()), "entries": int(ratio.size)}


def parity_sample_paged(w, inputs, out, n=6):
    """Max abs error of sampled output rows of a paged workload against the CPU oracle."""
    import numpy as np

    import oracle

    q, kp, vp, table, lens = inputs
    o, lse = out
    rng = np.random.default_rng(w.seed + 1)
    eo = el = 0.0
    for _ in range(n):
        b, h, i = int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.Nq))
        c = -(-int(lens[b]) // w.block_size)
        used = table[b, :c]
        ob, lb = oracle.paged_attention_forward(
            oracle.decode(q[b:b + 1, h:h + 1, i:i + 1], w.dtype), oracle.decode(kp[used, h:h + 1], w.dtype),
            oracle.decode(vp[used, h:h + 1], w.dtype), np.arange(c)[None], lens[b:b + 1], scale=w.scale)
        eo = max(eo, float(np.max(np.abs(o[b, h, i].float().cpu().numpy() - ob[0, 0, 0]))))
        el = max(el, abs(float(lse[b, h, i]) - float(lb[0, 0, 0])))
    return {"max_abs_dO": eo, "max_abs_dLSE": el, "rows": n}


def parity_sample(w, inputs, out, n=24):
    """Max abs error of sampled output rows against the CPU oracle."""
    import numpy as np
    import torch

    import oracle

    q, k, v = inputs
    o, lse = out
    rng = np.random.default_rng(123)
    picks = [(int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.N))) for _ in range(n)]
    picks += [(0, 0, 0), (w.B - 1, w.H - 1, w.N - 1)]
    picks = sorted(set(picks))
    o_ref, l_ref = oracle.attention_rows(q, k, v, causal=w.causal, scale=w.scale, picks=picks, dtype=w.dtype)
    idx = torch.tensor(picks, dtype=torch.long, device=o.device)
    og = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy()
    lg = lse[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy()
    return dict(rows=len(picks), max_abs_dO=float(np.max(np.abs(og - o_ref))),
                max_abs_dLSE=float(np.max(np.abs(lg - l_ref))))


def cpu_baseline(w, inputs, seconds):
    """The oracle as it stands on the host cores, over whole heads of the workload
    until about `seconds` of work; reported in the metric's unit (credited TFLOP/s)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    q, k, v = inputs
    affinity = len(os.sched_getaffinity(0))
    cores = host_workers()
    heads_per_call = max(1, min(w.H, math.ceil(cores / max(1, math.ceil(w.N / 1024)))))
    done_heads, t0 = 0, time.perf_counter()
    outs = []
    with threadpool_limits(limits=1):
        while True:
            b, h0 = divmod(done_heads, w.H)
            if b >= w.B:
                break
            h1 = min(w.H, h0 + heads_per_call)
            sl = (slice(b, b + 1), slice(h0, h1))
            outs.append((b, h0, h1) + oracle.attention_forward(
                oracle.decode(q[sl], w.dtype), oracle.decode(k[sl], w.dtype), oracle.decode(v[sl], w.dtype),
                causal=w.causal, scale=w.scale, threads=cores))
            done_heads += h1 - h0
            if time.perf_counter() - t0 >= seconds:
                break
    el = time.perf_counter() - t0
    flops = w.credited_flops() / (w.B * w.H) * done_heads
    res = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"{done_heads} of {w.B * w.H} heads (b, h in order) of {w.name}, float64, "
                     f"{el:.1f} s wall, numpy/OpenBLAS 1 thread per worker x {cores} workers "
                     f"({affinity} cores in the affinity mask)"}
    return res, outs


def host_workers() -> int:
    """Worker threads for the host oracle: every core of the affinity mask, capped by the
    CPU share the runtime grants this process (OMP_NUM_THREADS when set; one GPU's share
    of a shared host is 16 cores)."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def parity_full(w, out, oracle_heads):
    """Max abs error over every output element of the heads the CPU oracle evaluated."""
    import numpy as np

    o, lse = out
    eo = el = 0.0
    rows = 0
    for b, h0, h1, o_ref, l_ref in oracle_heads:
        og = o[b, h0:h1].float().cpu().numpy().astype(np.float64)
        lg = lse[b, h0:h1].cpu().numpy().astype(np.float64)
        eo = max(eo, float(np.max(np.abs(og - o_ref[0]))))
        el = max(el, float(np.max(np.abs(lg - l_ref[0]))))
        rows += (h1 - h0) * w.N
    return {"rows": rows, "of_rows": w.B * w.H * w.N, "max_abs_dO": eo, "max_abs_dLSE": el}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    # before the counted warm-up: launches for this many seconds, so that the clock has
    # reached the level it holds under sustained load whatever --warmup is
    ap.add_argument("--settle-seconds", type=float, default=1.5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="also time every workload (lines on stderr)")
    ap.add_argument("--decode", action="store_true",
                    help="also time the split-KV decode workloads (lines on stderr)")
    ap.add_argument("--gemm", action="store_true",
                    help="also time the dense GEMM workloads, with torch.matmul beside them (lines on stderr)")
    ap.add_argument("--paged", action="store_true",
                    help="also time the paged split-KV decode workloads (lines on stderr)")
    ap.add_argument("--pages-sweep", action="store_true",
                    help="also time the fp16 sweep of the paper's FlashAttention-2 figures (lines on stderr)")
    ap.add_argument("--vs-torch", action="store_true",
                    help="also time torch's fused attention (flash backend) beside this library on the "
                         "16-bit workloads (lines on stderr)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 device-to-device copies of BYTES bytes (to scale HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the fused forward runs on a single MI355X; "
              "multi-GPU runs are not part of this benchmark", file=sys.stderr)
        sys.exit(2)

    import torch

    import head_attention_fa2_amd as mha
    import mha_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mha.load()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # A plain copy of known size: FETCH_SIZE should read and WRITE_SIZE should
        # write exactly BYTES per launch; the ratio calibrates the counters.
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "launches": 5}))
        return
    w = mha_inputs.WORKLOADS[args.workload]

    r = time_gpu(w, args.steps, args.warmup, dev, settle_s=args.settle_seconds)
    ms = r["total_ms"] / args.steps
    flops = w.credited_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    avg_launch_ms = sum(r["per_ms"]) / len(r["per_ms"])
    median_launch_ms = sorted(r["per_ms"])[len(r["per_ms"]) // 2]
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    ctr = recorded_counters(w.name)
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "seed": w.seed, "pct_of_bf16_peak": round(100 * tflops / peak, 2)},
        "settle": r["settle"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": ctr["traffic_bytes"],
                     "kernel": f"mha_fwd_kernel<{w.dtype},{w.d},{'causal' if w.causal else 'full'}>",
                     "avg_launch_ms": round(avg_launch_ms, 5),
                     "median_launch_ms": round(median_launch_ms, 5),
                     "median_tflops": round(flops / (median_launch_ms * 1e-3) / 1e12, 2),
                     "mfma_busy": ctr["mfma_busy"], "hbm_gbs": ctr["hbm_gbs"],
                     "algorithmic_bytes": mha.mha_fwd_bytes(w.B, w.H, w.N, w.d, 1 if w.dtype == "bf16" else 0)},
    }
    oracle_heads = []
    if not args.no_cpu_baseline:
        line["cpu_baseline"], oracle_heads = cpu_baseline(w, r["inputs"], args.cpu_seconds)
    if not args.no_parity:
        # every element of the heads the CPU baseline evaluated, else sampled rows
        line["parity"] = parity_full(w, r["out"], oracle_heads) if oracle_heads else \
            parity_sample(w, r["inputs"], r["out"])
    del r, oracle_heads
    if args.sweep:
        for name, ww in mha_inputs.WORKLOADS.items():
            rr = time_gpu(ww, max(5, args.steps // 2), 3, dev, settle_s=0.5)
            m = rr["total_ms"] / max(5, args.steps // 2)
            tf = ww.credited_flops() / (m * 1e-3) / 1e12
            print(json.dumps({"workload": name, "ms": round(m, 5), "TFLOP/s": round(tf, 2),
                              "pct_of_peak": round(100 * tf / PEAK_TFLOPS["bf16"], 2),
                              "parity": parity_sample(ww, rr["inputs"], rr["out"], n=8)}),
                  file=sys.stderr, flush=True)
            del rr
    if args.decode:
        for name, ww in mha_inputs.DECODE.items():
            steps = max(10, args.steps // 2)
            rr = time_gpu_splitkv(ww, steps, 10, dev)
            m = rr["total_ms"] / steps
            nbytes = mha.mha_fwd_splitkv_bytes(ww.B, ww.H, ww.N, ww.Nk, ww.d,
                                               {"f32": 0, "bf16": 1, "f16": 2}[ww.dtype])
            print(json.dumps({"workload": name, "B": ww.B, "H": ww.H, "Nq": ww.N, "Nk": ww.Nk, "d": ww.d,
                              "splits": mha.mha_fwd_splitkv_splits(ww.B, ww.H, ww.N, ww.Nk, 0),
                              "ms": round(m, 5), "GB/s": round(nbytes / (m * 1e-3) / 1e9, 1),
                              "pct_of_hbm": round(100 * nbytes / (m * 1e-3) / 1e9 / HBM_GBS, 2),
                              "TFLOP/s": round(ww.credited_flops() / (m * 1e-3) / 1e12, 2),
                              "parity": parity_sample(ww, rr["inputs"], rr["out"], n=8)}),
                  file=sys.stderr, flush=True)
            del rr
    if args.gemm:
        for name, ww in mha_inputs.GEMM.items():
            rr = time_gemm(ww, max(10, args.steps // 4), 20, dev)
            tf = ww.flops() / (rr["ms"] * 1e-3) / 1e12
            tft = ww.flops() / (rr["ms_torch"] * 1e-3) / 1e12
            print(json.dumps({"workload": name, "M": ww.M, "N": ww.N, "K": ww.K, "ms": round(rr["ms"], 5),
                              "TFLOP/s": round(tf, 1), "pct_of_peak": round(100 * tf / PEAK_TFLOPS[ww.dtype], 2),
                              "torch_matmul_TFLOP/s": round(tft, 1), "vs_torch": round(tf / tft, 3),
                              "parity": parity_sample_gemm(ww, rr["inputs"], rr["out"])}),
                  file=sys.stderr, flush=True)
            del rr
    if args.gemm:
        for name, ww in mha_inputs.GEMM_MEMBOUND.items():
            rr = time_gemm_splitk(ww, max(10, args.steps // 4), 5, dev)
            nbytes = mha.mha_gemm_bytes(ww.M, ww.N, ww.K, {"bf16": 1, "f16": 2}[ww.dtype])
            gbs = nbytes / (rr["ms"] * 1e-3) / 1e9
            print(json.dumps({"workload": name, "M": ww.M, "N": ww.N, "K": ww.K,
                              "splits": mha.mha_gemm_splitk_splits(ww.M, ww.N, ww.K, 0), "ms": round(rr["ms"], 5),
                              "GB/s": round(gbs, 1), "pct_of_hbm": round(100 * gbs / HBM_GBS, 2),
                              "plain_gemm_GB/s": round(nbytes / (rr["ms_plain"] * 1e-3) / 1e9, 1),
                              "torch_matmul_GB/s": round(nbytes / (rr["ms_torch"] * 1e-3) / 1e9, 1),
                              "parity": parity_sample_gemm(ww, rr["inputs"], rr["out"])}),
                  file=sys.stderr, flush=True)
            del rr
    if args.paged:
        for name, ww in mha_inputs.PAGED.items():
            steps = max(10, args.steps // 2)
            rr = time_gpu_paged(ww, steps, 10, dev)
            m = rr["total_ms"] / steps
            table, lens = rr["inputs"][3], rr["inputs"][4]
            total_keys = int(lens.sum())
            nbytes = mha.mha_fwd_paged_bytes(ww.B, ww.H, ww.Nq, total_keys, ww.d,
                                             {"f32": 0, "bf16": 1, "f16": 2}[ww.dtype])
            print(json.dumps({"workload": name, "B": ww.B, "H": ww.H, "Nq": ww.Nq, "d": ww.d,
                              "block_size": ww.block_size, "total_keys": total_keys,
                              "splits": mha.mha_fwd_paged_splits(ww.B, ww.H, ww.Nq, ww.block_size, table.shape[1], 0),
                              "ms": round(m, 5), "GB/s": round(nbytes / (m * 1e-3) / 1e9, 1),
                              "pct_of_hbm": round(100 * nbytes / (m * 1e-3) / 1e9 / HBM_GBS, 2),
                              "parity": parity_sample_paged(ww, rr["inputs"], rr["out"])}),
                  file=sys.stderr, flush=True)
            del rr
    if args.pages_sweep:
        for name, ww in mha_inputs.SWEEP.items():
            steps = max(5, args.steps // 4)
            # each shape settles the clock at its own load first: a long shape before a
            # short one leaves the clock where the short one would not hold it
            rr = time_gpu(ww, steps, 5, dev, settle_s=0.5)
            m = rr["total_ms"] / steps
            tf = ww.credited_flops() / (m * 1e-3) / 1e12
            print(json.dumps({"workload": name, "B": ww.B, "H": ww.H, "N": ww.N, "d": ww.d,
                              "causal": ww.causal, "ms": round(m, 5), "TFLOP/s": round(tf, 2),
                              "pct_of_peak": round(100 * tf / PEAK_TFLOPS[ww.dtype], 2),
                              "parity": parity_sample(ww, rr["inputs"], rr["out"], n=8)}),
                  file=sys.stderr, flush=True)
            del rr
    if args.vs_torch:
        for name, ww in mha_inputs.WORKLOADS.items():
            if ww.dtype == "f32":
                continue
            rr = time_vs_torch(ww, 5, max(5, args.steps // 10), dev)
            out = {"workload": name}
            if rr.get("ms"):
                tf = ww.credited_flops() / (rr["ms"] * 1e-3) / 1e12
                tft = ww.credited_flops() / (rr["torch_flash_ms"] * 1e-3) / 1e12
                out.update({"TFLOP/s": round(tf, 1), "torch_flash_TFLOP/s": round(tft, 1),
                            "vs_torch": round(tf / tft, 3), "max_abs_diff_O": rr["max_abs_diff_O"]})
            else:
                out.update(rr)
            print(json.dumps(out), file=sys.stderr, flush=True)
            del rr
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
