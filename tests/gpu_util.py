"""Helpers for GPU tests: move seeded inputs to the device and outputs back."""
import os

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import head_attention_fa2_amd as mha
import mha_inputs
import oracle

# (O, LSE) max abs error.  fp16 has unit roundoff 2^-11: rounding P and O costs at
# most ~2 * 2^-11 * max|V| ~ 4e-3 for the N(0,1) values drawn here, so 5e-3.
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-3), "f16": (5e-3, 1e-3)}


def to_device(a: np.ndarray, dtype: str, dev="cuda:0"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def run(q, k, v, dtype, causal, scale=None, stream=None):
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    o, lse = mha.fwd(tq, tk, tv, causal=causal, scale=scale, stream=stream)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def host_threads() -> int:
    """Threads for the host oracle: the affinity mask, capped by the CPU share the
    runtime grants (OMP_NUM_THREADS when set)."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(share)) if share.isdigit() and int(share) > 0 else n)


def oracle_full(q, k, v, dtype, causal, scale, threads=1):
    """The float64 oracle over whole tensors; with threads > 1 the (batch, head, row-chunk)
    items run on a thread pool with one BLAS thread each."""
    args = (oracle.decode(q, dtype), oracle.decode(k, dtype), oracle.decode(v, dtype))
    if threads <= 1:
        return oracle.attention_forward(*args, causal=causal, scale=scale)
    with threadpool_limits(limits=1):
        return oracle.attention_forward(*args, causal=causal, scale=scale, threads=threads)


def draw(B, H, N, d, dtype, seed, qk_sigma=1.0, v_uniform=False):
    return mha_inputs.draw((B, H, N, d), dtype, seed, mha_inputs.Dist("normal", qk_sigma),
                           mha_inputs.Dist("uniform", -1.0, 1.0) if v_uniform else mha_inputs.Dist("normal", 1.0))
