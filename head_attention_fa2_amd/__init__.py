"""Fused multi-head attention forward (FlashAttention-2 style) for AMD MI355X.

The compute is entirely in ``libmha.so`` (hand-written HIP kernels for gfx950 behind
the C ABI of ``include/mha.h``).  This module only marshals arguments: the functions
``mha_fwd``, ``mha_fwd_validate``, ``mha_fwd_flops``, ``mha_fwd_bytes``,
``mha_fwd_splitkv``, ``mha_fwd_splitkv_validate``, ``mha_fwd_splitkv_splits``,
``mha_fwd_splitkv_workspace_size``, ``mha_fwd_splitkv_bytes``, ``mha_fwd_paged``,
``mha_fwd_paged_validate``, ``mha_fwd_paged_splits``, ``mha_fwd_paged_workspace_size``,
``mha_fwd_paged_bytes``, ``mha_gemm``, ``mha_gemm_validate``, ``mha_gemm_splitk``,
``mha_gemm_splitk_validate``, ``mha_gemm_splitk_splits``, ``mha_gemm_splitk_workspace_size``,
``mha_gemm_flops``, ``mha_gemm_bytes``, ``mha_status_string`` and ``mha_version`` mirror
the C entry points one to one, and :func:`fwd` / :func:`fwd_splitkv` / :func:`fwd_paged` /
:func:`gemm` / :func:`gemm_splitk` are the PyTorch-facing conveniences (device memory
and the stream
come from torch; nothing is computed in Python).  There is no fallback: if the library is not
built or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "MHA_OK", "MHA_ERR_INVALID_ARG", "MHA_ERR_UNSUPPORTED", "MHA_ERR_HIP", "MHA_ERR_SCRATCH",
    "MHA_SCRATCH_BYTES", "mha_fwd_splitkv_noalloc",
    "MHA_DTYPE_F32", "MHA_DTYPE_BF16", "MHA_DTYPE_F16",
    "library_path", "serial_library_path", "load", "load_serial", "mha_fwd", "mha_fwd_validate", "mha_fwd_flops",
    "mha_fwd_bytes", "mha_fwd_splitkv", "mha_fwd_splitkv_validate", "mha_fwd_splitkv_splits",
    "mha_fwd_splitkv_workspace_size", "mha_fwd_splitkv_bytes", "mha_fwd_paged", "mha_fwd_paged_validate",
    "mha_fwd_paged_splits", "mha_fwd_paged_workspace_size", "mha_fwd_paged_bytes", "mha_status_string",
    "mha_version", "mha_gemm", "mha_gemm_validate", "mha_gemm_splitk", "mha_gemm_splitk_validate",
    "mha_gemm_splitk_splits", "mha_gemm_splitk_workspace_size", "mha_gemm_flops", "mha_gemm_bytes",
    "fwd", "fwd_splitkv", "fwd_paged", "gemm", "gemm_splitk", "MhaError",
]

MHA_OK, MHA_ERR_INVALID_ARG, MHA_ERR_UNSUPPORTED, MHA_ERR_HIP, MHA_ERR_SCRATCH = 0, 1, 2, 3, 4
MHA_SCRATCH_BYTES = 16 << 20    # the static scratch of mha_fwd_splitkv_noalloc (include/mha.h)
MHA_DTYPE_F32, MHA_DTYPE_BF16, MHA_DTYPE_F16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None
_LIB_SERIAL: Optional[ctypes.CDLL] = None


class MhaError(RuntimeError):
    """A non-zero mha_status from the library."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(mha_status_string(status))


def library_path() -> str:
    return os.path.join(_HERE, "libmha.so")


def serial_library_path() -> str:
    return os.path.join(_HERE, "libmha_serial.so")


def load() -> ctypes.CDLL:
    """Load libmha.so (built in place by ``head_attention_fa2_amd.build``)."""
    global _LIB
    if _LIB is None:
        _LIB = _open(library_path())
    return _LIB


def load_serial() -> ctypes.CDLL:
    """Load libmha_serial.so: the same C ABI built with MHA_SERIALIZE=1 (the race-check
    form of the LDS tile loops, whose results must equal libmha.so's bit for bit).  For
    tests; the functions of this module always call libmha.so."""
    global _LIB_SERIAL
    if _LIB_SERIAL is None:
        _LIB_SERIAL = _open(serial_library_path())
    return _LIB_SERIAL


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with head_attention_fa2_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.mha_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.mha_fwd.restype = i
    lib.mha_fwd_validate.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i]
    lib.mha_fwd_validate.restype = i
    lib.mha_fwd_flops.argtypes = [i, i, i, i, i]
    lib.mha_fwd_flops.restype = ctypes.c_double
    lib.mha_fwd_bytes.argtypes = [i, i, i, i, i]
    lib.mha_fwd_bytes.restype = ctypes.c_double
    sz = ctypes.c_size_t
    lib.mha_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.mha_fwd_splitkv.restype = i
    lib.mha_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.mha_fwd_splitkv_noalloc.restype = i
    lib.mha_fwd_splitkv_validate.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz]
    lib.mha_fwd_splitkv_validate.restype = i
    lib.mha_fwd_splitkv_splits.argtypes = [i, i, i, i, i]
    lib.mha_fwd_splitkv_splits.restype = i
    lib.mha_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.mha_fwd_splitkv_workspace_size.restype = sz
    lib.mha_fwd_splitkv_bytes.argtypes = [i, i, i, i, i, i]
    lib.mha_fwd_splitkv_bytes.restype = ctypes.c_double
    lib.mha_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.mha_fwd_paged.restype = i
    lib.mha_fwd_paged_validate.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz]
    lib.mha_fwd_paged_validate.restype = i
    lib.mha_fwd_paged_splits.argtypes = [i, i, i, i, i, i]
    lib.mha_fwd_paged_splits.restype = i
    lib.mha_fwd_paged_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.mha_fwd_paged_workspace_size.restype = sz
    lib.mha_fwd_paged_bytes.argtypes = [i, i, i, ctypes.c_longlong, i, i]
    lib.mha_fwd_paged_bytes.restype = ctypes.c_double
    lib.mha_gemm.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.mha_gemm.restype = i
    lib.mha_gemm_validate.argtypes = [vp, vp, vp, i, i, i, i]
    lib.mha_gemm_validate.restype = i
    lib.mha_gemm_splitk.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz, vp]
    lib.mha_gemm_splitk.restype = i
    lib.mha_gemm_splitk_validate.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz]
    lib.mha_gemm_splitk_validate.restype = i
    lib.mha_gemm_splitk_splits.argtypes = [i, i, i, i]
    lib.mha_gemm_splitk_splits.restype = i
    lib.mha_gemm_splitk_workspace_size.argtypes = [i, i, i, i]
    lib.mha_gemm_splitk_workspace_size.restype = sz
    lib.mha_gemm_flops.argtypes = [i, i, i]
    lib.mha_gemm_flops.restype = ctypes.c_double
    lib.mha_gemm_bytes.argtypes = [i, i, i, i]
    lib.mha_gemm_bytes.restype = ctypes.c_double
    lib.mha_status_string.argtypes = [i]
    lib.mha_status_string.restype = ctypes.c_char_p
    lib.mha_version.argtypes = []
    lib.mha_version.restype = ctypes.c_char_p
    return lib


# ---------------------------------------------------------------- C entry points, 1:1
def mha_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int,
            causal: int, scale: float, dtype: int, stream: int) -> int:
    """Enqueue the fused forward on ``stream``; pointers are device addresses (ints)."""
    return load().mha_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream)


def mha_fwd_validate(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int,
                     causal: int, scale: float, dtype: int) -> int:
    return load().mha_fwd_validate(q, k, v, o, lse, B, H, N, d, causal, scale, dtype)


def mha_fwd_flops(B: int, H: int, N: int, d: int, causal: int) -> float:
    return load().mha_fwd_flops(B, H, N, d, causal)


def mha_fwd_bytes(B: int, H: int, N: int, d: int, dtype: int) -> float:
    return load().mha_fwd_bytes(B, H, N, d, dtype)


def mha_fwd_splitkv(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int, Nk: int,
                    d: int, scale: float, dtype: int, splits: int, workspace: int,
                    workspace_bytes: int, stream: int) -> int:
    """Enqueue the split-KV forward (partials, then the merge) on ``stream``."""
    return load().mha_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, dtype, splits,
                                  workspace, workspace_bytes, stream)


def mha_fwd_splitkv_noalloc(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int, Nk: int,
                            d: int, scale: float, dtype: int, splits: int, stream: int) -> int:
    """mha_fwd_splitkv with the partial results in the library's static device scratch
    (no workspace, no allocation); pointers are device addresses (ints)."""
    return load().mha_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, dtype, splits, stream)


def mha_fwd_splitkv_validate(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int,
                             Nk: int, d: int, scale: float, dtype: int, splits: int,
                             workspace: int, workspace_bytes: int) -> int:
    return load().mha_fwd_splitkv_validate(q, k, v, o, lse, B, H, Nq, Nk, d, scale, dtype, splits,
                                           workspace, workspace_bytes)


def mha_fwd_splitkv_splits(B: int, H: int, Nq: int, Nk: int, splits: int) -> int:
    return load().mha_fwd_splitkv_splits(B, H, Nq, Nk, splits)


def mha_fwd_splitkv_workspace_size(B: int, H: int, Nq: int, Nk: int, d: int, splits: int) -> int:
    return load().mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, splits)


def mha_fwd_splitkv_bytes(B: int, H: int, Nq: int, Nk: int, d: int, dtype: int) -> float:
    return load().mha_fwd_splitkv_bytes(B, H, Nq, Nk, d, dtype)


def mha_fwd_paged(q: int, k_pool: int, v_pool: int, block_table: int, seq_lens: int, o: int, lse: int,
                  B: int, H: int, Nq: int, d: int, num_blocks: int, block_size: int, max_blocks: int,
                  scale: float, dtype: int, splits: int, workspace: int, workspace_bytes: int,
                  stream: int) -> int:
    """Enqueue the paged split-KV forward (partials, then the merge) on ``stream``."""
    return load().mha_fwd_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H, Nq, d, num_blocks,
                                block_size, max_blocks, scale, dtype, splits, workspace, workspace_bytes,
                                stream)


def mha_fwd_paged_validate(q: int, k_pool: int, v_pool: int, block_table: int, seq_lens: int, o: int,
                           lse: int, B: int, H: int, Nq: int, d: int, num_blocks: int, block_size: int,
                           max_blocks: int, scale: float, dtype: int, splits: int, workspace: int,
                           workspace_bytes: int) -> int:
    return load().mha_fwd_paged_validate(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H, Nq, d,
                                         num_blocks, block_size, max_blocks, scale, dtype, splits, workspace,
                                         workspace_bytes)


def mha_fwd_paged_splits(B: int, H: int, Nq: int, block_size: int, max_blocks: int, splits: int) -> int:
    return load().mha_fwd_paged_splits(B, H, Nq, block_size, max_blocks, splits)


def mha_fwd_paged_workspace_size(B: int, H: int, Nq: int, d: int, block_size: int, max_blocks: int,
                                 splits: int) -> int:
    return load().mha_fwd_paged_workspace_size(B, H, Nq, d, block_size, max_blocks, splits)


def mha_fwd_paged_bytes(B: int, H: int, Nq: int, total_keys: int, d: int, dtype: int) -> float:
    return load().mha_fwd_paged_bytes(B, H, Nq, total_keys, d, dtype)


def mha_gemm(a: int, b: int, c: int, M: int, N: int, K: int, dtype: int, stream: int) -> int:
    """Enqueue C = A.B on ``stream``."""
    return load().mha_gemm(a, b, c, M, N, K, dtype, stream)


def mha_gemm_validate(a: int, b: int, c: int, M: int, N: int, K: int, dtype: int) -> int:
    return load().mha_gemm_validate(a, b, c, M, N, K, dtype)


def mha_gemm_splitk(a: int, b: int, c: int, M: int, N: int, K: int, dtype: int, splits: int, workspace: int,
                    workspace_bytes: int, stream: int) -> int:
    """Enqueue the split-K C = A.B (partials, then their sum) on ``stream``."""
    return load().mha_gemm_splitk(a, b, c, M, N, K, dtype, splits, workspace, workspace_bytes, stream)


def mha_gemm_splitk_validate(a: int, b: int, c: int, M: int, N: int, K: int, dtype: int, splits: int,
                             workspace: int, workspace_bytes: int) -> int:
    return load().mha_gemm_splitk_validate(a, b, c, M, N, K, dtype, splits, workspace, workspace_bytes)


def mha_gemm_splitk_splits(M: int, N: int, K: int, splits: int) -> int:
    return load().mha_gemm_splitk_splits(M, N, K, splits)


def mha_gemm_splitk_workspace_size(M: int, N: int, K: int, splits: int) -> int:
    return load().mha_gemm_splitk_workspace_size(M, N, K, splits)


def mha_gemm_flops(M: int, N: int, K: int) -> float:
    return load().mha_gemm_flops(M, N, K)


def mha_gemm_bytes(M: int, N: int, K: int, dtype: int) -> float:
    return load().mha_gemm_bytes(M, N, K, dtype)


def mha_status_string(status: int) -> str:
    return load().mha_status_string(status).decode()


def mha_version() -> str:
    return load().mha_version().decode()


# ---------------------------------------------------------------- torch convenience
def fwd(q, k, v, causal: bool = False, scale: Optional[float] = None, out=None, lse=None,
        stream=None) -> Tuple["object", "object"]:
    """``O, LSE = fwd(q, k, v)`` for contiguous ``[B, H, N, d]`` CUDA tensors.

    ``q, k, v``: float32, bfloat16 or float16, same shape, dtype and device.  ``scale`` defaults
    to 1/sqrt(d).  ``out`` / ``lse`` may be given to reuse buffers.  The kernel is
    enqueued on ``stream`` (default: torch's current stream of q's device); the call
    does not synchronise.
    """
    import torch

    _DTYPES = {torch.float32: MHA_DTYPE_F32, torch.bfloat16: MHA_DTYPE_BF16, torch.float16: MHA_DTYPE_F16}
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must have the same shape")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or len({q.device, k.device, v.device}) != 1:
        raise ValueError("q, k, v must be on the same GPU")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float32, all bfloat16 or all float16")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dtype = _DTYPES[q.dtype]
    with torch.cuda.device(q.device):
        rc = mha_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     B, H, N, d, int(bool(causal)), float(scale), dtype, stream.cuda_stream)
    if rc != MHA_OK:
        raise MhaError(rc)
    return out, lse


def fwd_splitkv(q, k, v, scale: Optional[float] = None, splits: int = 0, out=None, lse=None,
                workspace=None, stream=None) -> Tuple["object", "object"]:
    """``O, LSE = fwd_splitkv(q, k, v)``: ``q`` ``[B, H, Nq, d]`` against ``k, v``
    ``[B, H, Nk, d]`` (contiguous CUDA tensors of one dtype), no mask, with the keys cut
    into ``splits`` ranges (0: the library's choice).  ``workspace`` (a CUDA tensor of at
    least :func:`mha_fwd_splitkv_workspace_size` bytes) is allocated through torch when
    not given.  Enqueued on ``stream`` (default: torch's current stream); no sync.
    """
    import torch

    _DTYPES = {torch.float32: MHA_DTYPE_F32, torch.bfloat16: MHA_DTYPE_BF16, torch.float16: MHA_DTYPE_F16}
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d] with the batch, heads and d of q")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or len({q.device, k.device, v.device}) != 1:
        raise ValueError("q, k, v must be on the same GPU")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float32, all bfloat16 or all float16")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    need = mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = mha_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, H, Nq, Nk, d, float(scale), _DTYPES[q.dtype], int(splits),
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                         stream.cuda_stream)
    if st != MHA_OK:
        raise MhaError(st)
    return out, lse


def fwd_paged(q, k_pool, v_pool, block_table, seq_lens, scale: Optional[float] = None, splits: int = 0,
              out=None, lse=None, workspace=None, stream=None) -> Tuple["object", "object"]:
    """``O, LSE = fwd_paged(q, k_pool, v_pool, block_table, seq_lens)``: ``q``
    ``[B, H, Nq, d]`` against the keys of a paged cache, ``k_pool, v_pool``
    ``[num_blocks, H, block_size, d]`` (one dtype with q), ``block_table`` int32
    ``[B, max_blocks]`` and ``seq_lens`` int32 ``[B]``, all contiguous on one GPU.  Key j
    of sequence b is row ``j % block_size`` of block ``block_table[b, j // block_size]``.
    ``workspace`` as for :func:`fwd_splitkv` (size :func:`mha_fwd_paged_workspace_size`).
    Enqueued on ``stream`` (default: torch's current stream); no sync.
    """
    import torch

    _DTYPES = {torch.float32: MHA_DTYPE_F32, torch.bfloat16: MHA_DTYPE_BF16, torch.float16: MHA_DTYPE_F16}
    if q.dim() != 4 or k_pool.dim() != 4 or v_pool.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and the pools [num_blocks, H, block_size, d]")
    B, H, Nq, d = q.shape
    num_blocks, _, block_size, _ = k_pool.shape
    if k_pool.shape != (num_blocks, H, block_size, d) or v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool must be [num_blocks, H, block_size, d] with the heads and d of q")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    tensors = (q, k_pool, v_pool, block_table, seq_lens)
    if not all(t.is_cuda for t in tensors) or len({t.device for t in tensors}) != 1:
        raise ValueError("all inputs must be on the same GPU")
    if q.dtype not in _DTYPES or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("q and the pools must all be float32, all bfloat16 or all float16")
    if not all(t.is_contiguous() for t in tensors):
        raise ValueError("all inputs must be contiguous")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    need = mha_fwd_paged_workspace_size(B, H, Nq, d, block_size, max_blocks, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = mha_fwd_paged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
                       seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Nq, d, num_blocks,
                       block_size, max_blocks, float(scale), _DTYPES[q.dtype], int(splits),
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != MHA_OK:
        raise MhaError(st)
    return out, lse


def gemm(a, b, out=None, stream=None):
    """``C = gemm(a, b)``: ``a [M, K] @ b [K, N]`` for contiguous bfloat16 or float16 CUDA
    tensors of one dtype (float32 accumulation, C in the input dtype).  ``out`` may be
    given to reuse a buffer.  Enqueued on ``stream`` (default: torch's current stream);
    no sync.
    """
    import torch

    _DTYPES = {torch.bfloat16: MHA_DTYPE_BF16, torch.float16: MHA_DTYPE_F16}
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("need a [M, K] and b [K, N]")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    if a.dtype not in _DTYPES or b.dtype != a.dtype:
        raise ValueError("a and b must both be bfloat16 or both float16")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    M, K = a.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    elif out.shape != (M, N) or out.dtype != a.dtype or out.device != a.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor like a")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    st = mha_gemm(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, _DTYPES[a.dtype], stream.cuda_stream)
    if st != MHA_OK:
        raise MhaError(st)
    return out


def gemm_splitk(a, b, splits: int = 0, out=None, workspace=None, stream=None):
    """``C = gemm_splitk(a, b)``: as :func:`gemm`, with K cut into ``splits`` ranges (0:
    the library's choice) whose float32 partials are then summed; for shapes with one
    small dimension.  ``workspace`` (a CUDA tensor of at least
    :func:`mha_gemm_splitk_workspace_size` bytes) is allocated through torch when not given.
    """
    import torch

    _DTYPES = {torch.bfloat16: MHA_DTYPE_BF16, torch.float16: MHA_DTYPE_F16}
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("need a [M, K] and b [K, N]")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    if a.dtype not in _DTYPES or b.dtype != a.dtype:
        raise ValueError("a and b must both be bfloat16 or both float16")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    M, K = a.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    elif out.shape != (M, N) or out.dtype != a.dtype or out.device != a.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor like a")
    need = mha_gemm_splitk_workspace_size(M, N, K, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    elif not workspace.is_cuda or workspace.device != a.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor on a's device")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    st = mha_gemm_splitk(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, _DTYPES[a.dtype], int(splits),
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if st != MHA_OK:
        raise MhaError(st)
    return out
