"""mha_fwd_splitkv_noalloc (the split-KV forward with its partial results in the library's
static device scratch, for callers that cannot allocate) against mha_fwd_splitkv (the same
kernels with a caller workspace), through the C ABI: identical outputs bit for bit on two
calls in a row, the second with a smaller input, and a clear rejection of a call that
needs more than the scratch holds."""
import math

import pytest
import torch

import head_attention_fa2_amd as mha
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

_DT = {"bf16": mha.MHA_DTYPE_BF16, "f16": mha.MHA_DTYPE_F16, "f32": mha.MHA_DTYPE_F32}


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _case(B, H, Nq, Nk, d, dtype, seed):
    lib = mha.load()
    q, _, _ = gu.draw(B, H, Nq, d, dtype, seed=seed)
    _, k, v = gu.draw(B, H, Nk, d, dtype, seed=seed + 1)
    tq, tk, tv = (gu.to_device(x, dtype) for x in (q, k, v))
    scale = 1 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    need = mha.mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, 0)
    assert 0 < need <= mha.MHA_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=tq.device)
    o_ref, l_ref = torch.empty_like(tq), torch.empty((B, H, Nq), dtype=torch.float32, device=tq.device)
    rc = lib.mha_fwd_splitkv(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o_ref.data_ptr(), l_ref.data_ptr(),
                             B, H, Nq, Nk, d, scale, _DT[dtype], 0, ws.data_ptr(), need, stream)
    assert rc == mha.MHA_OK
    o = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), device=tq.device)
    rc = lib.mha_fwd_splitkv_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     B, H, Nq, Nk, d, scale, _DT[dtype], 0, stream)
    assert rc == mha.MHA_OK
    torch.cuda.synchronize()
    print(f"noalloc B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dtype}: workspace {need} bytes", flush=True)
    assert torch.equal(_bits(o), _bits(o_ref)) and torch.equal(lse.view(torch.int32), l_ref.view(torch.int32))
    # and within the oracle's tolerance (the outputs are the split-KV path's)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())


def test_noalloc_matches_workspace_entry_point_twice_second_smaller():
    _case(4, 8, 4, 40000, 128, "bf16", seed=61)      # 8+ splits, the larger call first
    _case(2, 3, 1, 3000, 64, "f16", seed=62)         # then a smaller one reusing the scratch


def test_noalloc_rejects_calls_beyond_the_scratch():
    lib = mha.load()
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    p = x.data_ptr()
    # 1024 heads x 300 query rows x 129 floats x splits > 16 MiB
    B, H, Nq, Nk, d = 64, 16, 300, 65536, 128
    assert mha.mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, 0) > mha.MHA_SCRATCH_BYTES
    rc = lib.mha_fwd_splitkv_noalloc(p, p, p, p, p, B, H, Nq, Nk, d, 0.1, mha.MHA_DTYPE_BF16, 0,
                                     torch.cuda.current_stream().cuda_stream)
    assert rc == mha.MHA_ERR_SCRATCH
    assert mha.mha_status_string(rc).startswith("MHA_ERR_SCRATCH")
