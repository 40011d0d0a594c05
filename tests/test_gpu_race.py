"""Race check of the LDS tile pipelines: libmha.so (double-buffered tiles, the copy of tile
t+1 in flight while tile t is read, one barrier per tile) against libmha_serial.so (the
same sources built with MHA_SERIALIZE=1: one buffer, every tile copied, waited for and
fenced by barriers before and after it is read).  The arithmetic and its order are the
same in both, so every output must be identical bit for bit; an ordering bug in the
pipeline (a tile read before its copy landed, or overwritten while still being read)
shows up as a difference.  Both libraries are called through the C ABI on the same
device buffers.

The loop being checked is the load/compute loop over K/V blocks of Algorithm 1
("FlashAttention-2 forward"), "ML-Triton, A Multi-Level Compilation and Language Extension
to Triton GPU Programming", section 2.5."""
import math

import numpy as np
import pytest
import torch

import head_attention_fa2_amd as mha
import mha_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

_DT = {"f32": mha.MHA_DTYPE_F32, "bf16": mha.MHA_DTYPE_BF16, "f16": mha.MHA_DTYPE_F16}


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same(a, b, what):
    diff = int((_bits(a) != _bits(b)).sum())
    print(f"{what}: {diff} differing elements of {a.numel()}", flush=True)
    assert diff == 0, what


def _stream():
    return torch.cuda.current_stream().cuda_stream


# Reduced forms of the benchmark workloads (several query blocks, ragged tails) plus the
# other element types and head sizes.
FWD = [
    ("bf16", 4, 8, 1024, 64, False),    # the B4 H16 N1024 d64 workload's shape class
    ("bf16", 2, 8, 1500, 128, True),    # the causal d128 workload at reduced size
    ("bf16", 1, 8, 2049, 128, False),
    ("f16", 2, 4, 777, 64, True),
    ("f16", 1, 4, 1100, 128, False),
    ("bf16", 1, 130, 256, 64, False),   # grids above the key-half threshold: 4-wavefront form
    ("f16", 1, 130, 300, 128, True),
    ("f32", 1, 2, 300, 64, False),
    ("f32", 1, 2, 200, 128, True),
]


@pytest.mark.parametrize("dtype,B,H,N,d,causal", FWD)
def test_fused_forward_serialized_equals_pipelined(dtype, B, H, N, d, causal):
    serial = mha.load_serial()
    q, k, v = gu.draw(B, H, N, d, dtype, seed=3000 + N + d, qk_sigma=2.0)
    tq, tk, tv = (gu.to_device(x, dtype) for x in (q, k, v))
    scale = 1 / math.sqrt(d)
    o1, l1 = mha.fwd(tq, tk, tv, causal=causal, scale=scale)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    rc = serial.mha_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                        B, H, N, d, int(causal), scale, _DT[dtype], _stream())
    assert rc == mha.MHA_OK
    torch.cuda.synchronize()
    _same(o1, o2, f"O {dtype} B{B} H{H} N{N} d{d} causal={causal}")
    _same(l1, l2, "LSE")


@pytest.mark.parametrize("dtype,d,Nq,Nk,splits", [("bf16", 128, 1, 5000, 0), ("f16", 64, 4, 3000, 3),
                                                  ("f32", 64, 2, 700, 2)])
def test_splitkv_serialized_equals_pipelined(dtype, d, Nq, Nk, splits):
    serial = mha.load_serial()
    B, H = 2, 3
    q, _, _ = gu.draw(B, H, Nq, d, dtype, seed=Nq + d)
    _, k, v = gu.draw(B, H, Nk, d, dtype, seed=Nk + d)
    tq, tk, tv = (gu.to_device(x, dtype) for x in (q, k, v))
    scale = 1 / math.sqrt(d)
    o1, l1 = mha.fwd_splitkv(tq, tk, tv, scale=scale, splits=splits)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    ws_bytes = mha.mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, splits)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=tq.device)
    rc = serial.mha_fwd_splitkv(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                                B, H, Nq, Nk, d, scale, _DT[dtype], splits, ws.data_ptr(), ws_bytes, _stream())
    assert rc == mha.MHA_OK
    torch.cuda.synchronize()
    _same(o1, o2, f"split-KV O {dtype} d{d} Nq{Nq} Nk{Nk}")
    _same(l1, l2, "split-KV LSE")


@pytest.mark.parametrize("block_size", [16, 64, 256])
def test_paged_serialized_equals_pipelined(block_size):
    serial = mha.load_serial()
    B, H, Nq, d = 3, 2, 2, 128
    lens = [700, 1, 300]
    q, kp, vp, table, lens_a = mha_inputs.draw_paged(B, H, Nq, d, "bf16", block_size, lens, seed=block_size)
    tq, tk, tv = (gu.to_device(x, "bf16") for x in (q, kp, vp))
    tt, tl = torch.from_numpy(table).cuda(), torch.from_numpy(lens_a).cuda()
    scale = 1 / math.sqrt(d)
    o1, l1 = mha.fwd_paged(tq, tk, tv, tt, tl, scale=scale)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    nb, mb = kp.shape[0], table.shape[1]
    ws_bytes = mha.mha_fwd_paged_workspace_size(B, H, Nq, d, block_size, mb, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=tq.device)
    rc = serial.mha_fwd_paged(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), tt.data_ptr(), tl.data_ptr(),
                              o2.data_ptr(), l2.data_ptr(), B, H, Nq, d, nb, block_size, mb, scale,
                              mha.MHA_DTYPE_BF16, 0, ws.data_ptr(), ws_bytes, _stream())
    assert rc == mha.MHA_OK
    torch.cuda.synchronize()
    _same(o1, o2, f"paged O bs{block_size}")
    _same(l1, l2, "paged LSE")


@pytest.mark.parametrize("M,N,K", [(300, 264, 200), (1024, 1024, 4096), (4096, 1024, 256)])
def test_gemm_serialized_equals_pipelined(M, N, K):
    serial = mha.load_serial()
    a, b = mha_inputs.draw_gemm(M, N, K, "bf16", seed=M + N + K)
    ta, tb = gu.to_device(a, "bf16"), gu.to_device(b, "bf16")
    c1 = mha.gemm(ta, tb)
    c2 = torch.full_like(c1, float("nan"))
    rc = serial.mha_gemm(ta.data_ptr(), tb.data_ptr(), c2.data_ptr(), M, N, K, mha.MHA_DTYPE_BF16, _stream())
    assert rc == mha.MHA_OK
    torch.cuda.synchronize()
    _same(c1, c2, f"GEMM M{M} N{N} K{K}")
    assert np.isfinite(c1.float().cpu().numpy()).all()
