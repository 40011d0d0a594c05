"""GPU parity of the dense GEMM (mha_gemm): C = A.B compared element by element with the
CPU oracle's float64 product, within the oracle's bound for a float32-accumulated,
once-rounded result (u_out |C| + gamma_K |A||B|, bf16 u = 2^-8, fp16 u = 2^-11).  The
element-wise shapes cover ragged M, N and K (partial tiles, K not a multiple of the
64-wide k-step) under the four tilings (256 x 256 from 192 such tiles, else 128 x 128
from 384 such tiles, else for K >= 2048 128 x 128 with the k-steps split between two
groups of wavefronts, else 128 x 64); the full-size workloads are checked on sampled rows
and columns."""
import numpy as np
import pytest
import torch

import head_attention_fa2_amd as mha
import mha_inputs
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _check(c, a, b, dtype, what):
    ref = oracle.gemm(a, b)
    bound = oracle.gemm_error_bound(a, b, dtype)
    err = np.abs(c - ref)
    worst = float(np.max(err / bound))
    print(f"{what}: max|dC|={float(err.max()):.3e}, max err/bound={worst:.3f}", flush=True)
    assert np.all(np.isfinite(c)), what
    assert np.all(err <= bound), what


def _run(a_bits, b_bits, dtype):
    ta, tb = gu.to_device(a_bits, dtype), gu.to_device(b_bits, dtype)
    c = mha.gemm(ta, tb)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


CASES = [
    # (M, N, K, dtype)
    (1, 8, 8, "bf16"), (256, 256, 64, "bf16"), (300, 520, 200, "bf16"), (512, 768, 1024, "bf16"),
    (33, 1000, 72, "f16"), (777, 264, 136, "bf16"), (1024, 1024, 8, "f16"), (257, 2056, 640, "f16"),
    (2048, 256, 4104, "bf16"), (96, 64, 4096, "bf16"),
    # 208 tiles of 256 x 256: the large tiling, ragged in M, N and K
    (4000, 3080, 1000, "bf16"), (3900, 3336, 264, "f16"),
    # 384-400 tiles of 128 x 128 (and under 192 large ones): the 128 x 128 tiling
    (2048, 3072, 264, "bf16"), (2000, 3080, 136, "f16"),
    # fewer than 384 tiles of 128 x 128 and K >= 2048: two k-groups per workgroup, with an
    # even, an odd and a ragged number of k-steps (the second group then has one fewer)
    (130, 4104, 2048, "bf16"), (1000, 1032, 2056, "f16"), (700, 520, 2112, "bf16"), (1024, 1024, 4160, "bf16"),
]


@pytest.mark.parametrize("M,N,K,dtype", CASES)
def test_gemm_elementwise(M, N, K, dtype):
    a_bits, b_bits = mha_inputs.draw_gemm(M, N, K, dtype, seed=M * 7 + N + K)
    c = _run(a_bits, b_bits, dtype)
    _check(c, oracle.decode(a_bits, dtype), oracle.decode(b_bits, dtype), dtype, f"gemm M{M} N{N} K{K} {dtype}")


def test_gemm_closed_forms():
    # all-ones operands: every entry is exactly K (representable); identity: C = A
    ones = np.ones((300, 136), dtype=np.float32)
    c = _run(mha_inputs.f32_to_bf16_bits(ones), mha_inputs.f32_to_bf16_bits(np.ones((136, 264), np.float32)), "bf16")
    assert np.all(c == 136.0)
    a_bits, _ = mha_inputs.draw_gemm(300, 8, 264, "bf16", seed=5)
    eye = mha_inputs.f32_to_bf16_bits(np.eye(264, dtype=np.float32))
    np.testing.assert_array_equal(_run(a_bits, eye, "bf16"), oracle.decode(a_bits, "bf16"))
    # the same with K long enough for two k-groups (each sums 2048 ones exactly)
    c = _run(mha_inputs.f32_to_bf16_bits(np.ones((200, 4096), np.float32)),
             mha_inputs.f32_to_bf16_bits(np.ones((4096, 136), np.float32)), "bf16")
    assert np.all(c == 4096.0)


def test_gemm_scaled_operands():
    # large and small magnitudes: the bound is relative, so both must hold
    for sigma in (100.0, 1e-3):
        a_bits, b_bits = mha_inputs.draw_gemm(384, 320, 512, "bf16", seed=int(sigma * 10) + 1,
                                              dist=mha_inputs.Dist("normal", sigma))
        c = _run(a_bits, b_bits, "bf16")
        _check(c, oracle.decode(a_bits, "bf16"), oracle.decode(b_bits, "bf16"), "bf16", f"sigma={sigma}")


@pytest.mark.parametrize("name", [n for n in mha_inputs.GEMM if "M16384" not in n or "N4096_K4096" in n])
def test_gemm_workload_sampled(name):
    w = mha_inputs.GEMM[name]
    a_bits, b_bits = mha_inputs.draw_gemm(w.M, w.N, w.K, w.dtype, w.seed)
    ta, tb = gu.to_device(a_bits, w.dtype), gu.to_device(b_bits, w.dtype)
    c = mha.gemm(ta, tb)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(c).all())
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([rng.integers(0, w.M, 12), [0, w.M - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, w.N, 12), [0, w.N - 1]]))
    cg = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].float().cpu().numpy().astype(np.float64)
    a = oracle.decode(a_bits[rows], w.dtype)
    b = oracle.decode(b_bits[:, cols], w.dtype)
    _check(cg, a, b, w.dtype, f"{name}, {len(rows)}x{len(cols)} sampled entries")


def test_gemm_errors_raise():
    a = torch.zeros(4, 12, device="cuda", dtype=torch.bfloat16)
    b = torch.zeros(12, 8, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(mha.MhaError) as e:
        mha.gemm(a, b)                         # K = 12 is not a multiple of 8
    assert e.value.status == mha.MHA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        mha.gemm(a, b[:8])
    with pytest.raises(ValueError):
        mha.gemm(a.float(), b.float())


SPLITK_CASES = [
    # (M, N, K, dtype, splits)
    (1, 8, 8, "bf16", 0), (16, 1000, 4104, "bf16", 0), (33, 264, 1000, "f16", 3), (300, 520, 200, "bf16", 2),
    (16, 4096, 2048, "bf16", 7), (129, 136, 8192, "f16", 0), (2, 64, 640, "bf16", 100),
]


@pytest.mark.parametrize("M,N,K,dtype,splits", SPLITK_CASES)
def test_gemm_splitk_elementwise(M, N, K, dtype, splits):
    a_bits, b_bits = mha_inputs.draw_gemm(M, N, K, dtype, seed=M * 3 + N + K + splits)
    ta, tb = gu.to_device(a_bits, dtype), gu.to_device(b_bits, dtype)
    c = mha.gemm_splitk(ta, tb, splits=splits)
    torch.cuda.synchronize()
    used = mha.mha_gemm_splitk_splits(M, N, K, splits)
    _check(c.float().cpu().numpy().astype(np.float64), oracle.decode(a_bits, dtype), oracle.decode(b_bits, dtype),
           dtype, f"gemm_splitk M{M} N{N} K{K} {dtype} splits={splits} (used {used})")


def test_gemm_splitk_workspace_reused():
    ws = torch.empty(mha.mha_gemm_splitk_workspace_size(64, 2048, 4096, 8), dtype=torch.uint8, device="cuda")
    for (M, N, K, splits) in ((64, 2048, 4096, 8), (16, 520, 1000, 3)):
        a_bits, b_bits = mha_inputs.draw_gemm(M, N, K, "bf16", seed=K + N)
        c = mha.gemm_splitk(gu.to_device(a_bits, "bf16"), gu.to_device(b_bits, "bf16"), splits=splits, workspace=ws)
        torch.cuda.synchronize()
        _check(c.float().cpu().numpy().astype(np.float64), oracle.decode(a_bits, "bf16"),
               oracle.decode(b_bits, "bf16"), "bf16", f"shared workspace M{M} N{N} K{K}")


@pytest.mark.parametrize("name", list(mha_inputs.GEMM_MEMBOUND))
def test_gemm_membound_workload(name):
    w = mha_inputs.GEMM_MEMBOUND[name]
    a_bits, b_bits = mha_inputs.draw_gemm(w.M, w.N, w.K, w.dtype, w.seed)
    ta, tb = gu.to_device(a_bits, w.dtype), gu.to_device(b_bits, w.dtype)
    c = mha.gemm_splitk(ta, tb)
    c2 = mha.gemm(ta, tb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([rng.integers(0, w.M, 12), [0, w.M - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, w.N, 12), [0, w.N - 1]]))
    a = oracle.decode(a_bits[rows], w.dtype)
    b = oracle.decode(b_bits[:, cols], w.dtype)
    for out, how in ((c, "split-K"), (c2, "plain")):
        cg = out[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].float().cpu().numpy()
        _check(cg.astype(np.float64), a, b, w.dtype,
               f"{name} {how}, splits {mha.mha_gemm_splitk_splits(w.M, w.N, w.K, 0)}")
