"""GPU parity of the split-KV forward (mha_fwd_splitkv): few query rows against a long
key/value sequence, keys cut into ranges whose partial results are merged.  Compared
element by element (small shapes) or on sampled rows (the decode workloads) with the
CPU oracle's plain definition over all keys.  Tolerances as for the fused kernel:
fp32 1e-4 / 1e-4, bf16 2e-2 / 1e-3, fp16 5e-3 / 1e-3 (max |dO|, max |dLSE|)."""
import math

import numpy as np
import pytest
import torch

import head_attention_fa2_amd as mha
import mha_inputs
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _draw(B, H, Nq, Nk, d, dtype, seed, sigma=1.0):
    return mha_inputs.draw((B, H, Nq, d), dtype, seed, mha_inputs.Dist("normal", sigma),
                           mha_inputs.Dist("normal", 1.0), kv_shape=(B, H, Nk, d))


def _run(q, k, v, dtype, scale, splits, workspace=None):
    tq, tk, tv = (gu.to_device(x, dtype) for x in (q, k, v))
    o, lse = mha.fwd_splitkv(tq, tk, tv, scale=scale, splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(o, lse, o_ref, l_ref, dtype, what):
    tol_o, tol_l = gu.TOL[dtype]
    eo, el = float(np.max(np.abs(o - o_ref))), float(np.max(np.abs(lse - l_ref)))
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    assert eo <= tol_o and el <= tol_l, what


CASES = [
    # (B, H, Nq, Nk, d, dtype, splits)
    (1, 1, 1, 1, 64, "bf16", 0), (1, 2, 1, 63, 128, "bf16", 0), (2, 1, 1, 65, 64, "f16", 2),
    (1, 3, 2, 1000, 128, "bf16", 3), (2, 2, 4, 4097, 128, "bf16", 0), (1, 2, 4, 4097, 64, "f16", 7),
    (1, 2, 33, 700, 128, "f32", 3), (1, 1, 1, 2048, 64, "f32", 0), (2, 2, 130, 1500, 64, "bf16", 4),
    (1, 4, 1, 5000, 128, "f16", 1000), (3, 2, 1, 3000, 128, "bf16", 1), (1, 1, 200, 200, 128, "bf16", 2),
    (2, 2, 5, 900, 64, "f32", 1), (1, 3, 130, 777, 64, "f16", 1),      # one range: no merge
    (1, 2, 1, 2100 * 64, 64, "bf16", 2100),   # more ranges than the merge keeps weights for in LDS
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,dtype,splits", CASES)
def test_splitkv_elementwise(B, H, Nq, Nk, d, dtype, splits):
    q, k, v = _draw(B, H, Nq, Nk, d, dtype, seed=600 + Nq + Nk + d, sigma=1.5)
    scale = 1 / math.sqrt(d)
    o, lse = _run(q, k, v, dtype, scale, splits)
    o_ref, l_ref = gu.oracle_full(q, k, v, dtype, False, scale)
    _check(o, lse, o_ref, l_ref, dtype, f"splitkv B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dtype} splits={splits}")


def test_splitkv_large_logits_and_scales():
    B, H, Nq, Nk, d = 1, 2, 3, 900, 64
    for sigma, scale in ((5.0, 0.5), (1.0, -0.3), (1.0, 0.0)):
        q, k, v = _draw(B, H, Nq, Nk, d, "bf16", seed=int(sigma * 10) + 7, sigma=sigma)
        o, lse = _run(q, k, v, "bf16", scale, 5)
        o_ref, l_ref = gu.oracle_full(q, k, v, "bf16", False, scale)
        _check(o, lse, o_ref, l_ref, "bf16", f"splitkv sigma={sigma} scale={scale}")


def test_splitkv_matches_fused_kernel_when_square():
    q, k, v = _draw(2, 3, 777, 777, 128, "bf16", seed=41)
    tq, tk, tv = (gu.to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = mha.fwd(tq, tk, tv, causal=False)
    o2, l2 = mha.fwd_splitkv(tq, tk, tv, splits=4)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-2
    assert float((l1 - l2).abs().max()) <= 1e-3


def test_splitkv_workspace_reused_by_consecutive_calls():
    ws = torch.empty(mha.mha_fwd_splitkv_workspace_size(2, 4, 3, 3000, 128, 6), dtype=torch.uint8, device="cuda")
    for (B, H, Nq, Nk, splits) in ((2, 4, 3, 3000, 6), (1, 2, 2, 700, 3)):
        q, k, v = _draw(B, H, Nq, Nk, 128, "bf16", seed=Nk)
        o, lse = _run(q, k, v, "bf16", 1 / math.sqrt(128), splits, workspace=ws)
        o_ref, l_ref = gu.oracle_full(q, k, v, "bf16", False, 1 / math.sqrt(128))
        _check(o, lse, o_ref, l_ref, "bf16", f"shared workspace Nk{Nk}")


@pytest.mark.parametrize("name", list(mha_inputs.DECODE))
def test_decode_workload_sampled(name):
    w = mha_inputs.DECODE[name]
    q, k, v = mha_inputs.draw_qkv(w)
    tq, tk, tv = (gu.to_device(x, w.dtype) for x in (q, k, v))
    o, lse = mha.fwd_splitkv(tq, tk, tv, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(w.seed)
    picks = sorted({(int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.N))) for _ in range(16)})
    picks += [(0, 0, 0), (w.B - 1, w.H - 1, w.N - 1)]
    o_ref, l_ref = oracle.attention_rows(q, k, v, causal=False, scale=w.scale, picks=picks, dtype=w.dtype)
    idx = torch.tensor(picks, dtype=torch.long, device=o.device)
    og = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy().astype(np.float64)
    lg = lse[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy().astype(np.float64)
    _check(og, lg, o_ref, l_ref, w.dtype, f"{name}, {len(picks)} sampled rows, "
           f"{mha.mha_fwd_splitkv_splits(w.B, w.H, w.N, w.Nk, 0)} splits")


def test_splitkv_errors_raise():
    q = torch.zeros(1, 1, 1, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 100, 64, device="cuda", dtype=torch.bfloat16)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(mha.MhaError) as e:
        mha.fwd_splitkv(q, k, k, workspace=small)
    assert e.value.status == mha.MHA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        mha.fwd_splitkv(q, k[:, :, :, :32], k)
