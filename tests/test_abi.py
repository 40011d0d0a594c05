"""The C-ABI library: it loads, exports every entry point include/mha.h declares, and
its host-side validation and accounting behave as documented.  No GPU work is
launched: every mha_fwd call here is rejected on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import head_attention_fa2_amd as mha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mha.h")

OK, INVALID, UNSUPPORTED = mha.MHA_OK, mha.MHA_ERR_INVALID_ARG, mha.MHA_ERR_UNSUPPORTED
BF16, F32, F16 = mha.MHA_DTYPE_BF16, mha.MHA_DTYPE_F32, mha.MHA_DTYPE_F16
P = 0x10000  # a 16-byte aligned fake address (never dereferenced by validation)


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mha_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = mha.load()
    names = declared_functions()
    assert {"mha_fwd", "mha_fwd_validate", "mha_fwd_flops", "mha_fwd_bytes",
            "mha_status_string", "mha_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
        assert hasattr(mha, name), name          # Python binding mirrors the C names


def test_exported_symbols_are_c_linkage():
    out = os.popen(f"nm -D --defined-only {mha.library_path()}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def v(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, causal=0, scale=0.125, dtype=BF16)
    a.update(kw)
    return mha.mha_fwd_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                                a["d"], a["causal"], a["scale"], a["dtype"])


def test_validate_accepts_good_arguments():
    assert v() == OK
    assert v(d=128, causal=1, dtype=F32) == OK
    assert v(d=128, causal=1, dtype=F16) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(v=0), INVALID), (dict(o=0), INVALID),
    (dict(lse=0), INVALID), (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(N=0), INVALID),
    (dict(causal=2), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(dtype=7), INVALID), (dict(dtype=3), INVALID),
    (dict(d=32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(q=P + 8), UNSUPPORTED), (dict(o=P + 4), UNSUPPORTED), (dict(lse=P + 2), UNSUPPORTED),
    (dict(B=65536, H=65536, N=1 << 20), UNSUPPORTED),
])
def test_validate_rejects(kw, code):
    assert v(**kw) == code


def test_mha_fwd_rejects_before_launch():
    # invalid arguments: mha_fwd returns the validation code and enqueues nothing
    assert mha.mha_fwd(0, P, P, P, P, 1, 1, 16, 64, 0, 0.125, BF16, 0) == INVALID
    assert mha.mha_fwd(P, P, P, P, P, 1, 1, 16, 80, 0, 0.125, BF16, 0) == UNSUPPORTED


def test_flops_and_bytes():
    assert mha.mha_fwd_flops(4, 32, 4096, 128, 1) == 4 * 4 * 32 * 4096 ** 2 * 128 / 2
    assert mha.mha_fwd_flops(4, 16, 1024, 64, 0) == 4 * 4 * 16 * 1024 ** 2 * 64
    assert mha.mha_fwd_bytes(4, 32, 4096, 128, BF16) == 4 * 4 * 32 * 4096 * 128 * 2 + 4 * 4 * 32 * 4096
    assert mha.mha_fwd_bytes(1, 2, 128, 64, F32) == 4 * 2 * 128 * 64 * 4 + 4 * 2 * 128
    assert mha.mha_fwd_bytes(2, 16, 1024, 128, F16) == 4 * 2 * 16 * 1024 * 128 * 2 + 4 * 2 * 16 * 1024


def test_status_strings():
    for code in (OK, INVALID, UNSUPPORTED, mha.MHA_ERR_HIP):
        s = mha.mha_status_string(code)
        assert s.startswith(["MHA_OK", "MHA_ERR_INVALID_ARG", "MHA_ERR_UNSUPPORTED", "MHA_ERR_HIP"][code])
    assert mha.mha_status_string(99) == "unknown mha_status"
    assert mha.mha_version().startswith("mha-gfx950")


def test_python_wrapper_checks_shapes_on_cpu():
    import torch
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        mha.fwd(q, q, q)                    # CPU tensors are refused before any call
    with pytest.raises(ValueError):
        mha.fwd(q[0], q[0], q[0])           # wrong rank


def sv(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=4, Nq=1, Nk=1000, d=128, scale=0.1, dtype=BF16,
             splits=0, ws=P, wsb=1 << 30)
    a.update(kw)
    return mha.mha_fwd_splitkv_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                        a["Nq"], a["Nk"], a["d"], a["scale"], a["dtype"], a["splits"],
                                        a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(dtype=F32, d=64), OK), (dict(dtype=F16, splits=5), OK),
    (dict(ws=0), INVALID), (dict(wsb=16), INVALID), (dict(Nq=0), INVALID), (dict(Nk=0), INVALID),
    (dict(splits=-1), INVALID), (dict(q=0), INVALID), (dict(dtype=3), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(d=96), UNSUPPORTED), (dict(ws=P + 4), UNSUPPORTED),
    (dict(k=P + 8), UNSUPPORTED),
])
def test_splitkv_validate(kw, code):
    assert sv(**kw) == code


def test_splitkv_rejects_before_launch():
    assert mha.mha_fwd_splitkv(P, P, P, P, P, 1, 1, 1, 100, 64, 0.1, BF16, 0, 0, 0, 0) == INVALID


@pytest.mark.parametrize("B,H,Nq,Nk", [(1, 1, 1, 1), (1, 32, 1, 16384), (16, 32, 1, 16384), (1, 8, 4, 131072),
                                        (3, 5, 130, 999), (64, 8, 1, 4096), (1, 1, 1, 100)])
@pytest.mark.parametrize("splits", [0, 1, 2, 7, 1000])
def test_splitkv_partition(B, H, Nq, Nk, splits):
    s = mha.mha_fwd_splitkv_splits(B, H, Nq, Nk, splits)
    tiles = -(-Nk // 64)
    assert 1 <= s <= tiles
    if splits > 0:
        assert s <= splits
    else:
        # about 512 workgroups, at least 512 keys per range (unless one range)
        blocks = -(-Nq // 128) * B * H
        assert s == 1 or (s - 1) * 512 < Nk
        assert s <= max(1, -(-512 // blocks))
    assert mha.mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, 128, splits) == s * B * H * Nq * 129 * 4
    assert mha.mha_fwd_splitkv_bytes(B, H, Nq, Nk, 128, BF16) == \
        (2 * Nq + 2 * Nk) * B * H * 128 * 2 + 4 * B * H * Nq


def pv(**kw):
    a = dict(q=P, kp=P, vp=P, bt=P, sl=P, o=P, lse=P, B=4, H=8, Nq=1, d=128, nb=100, bs=16, mb=64,
             scale=0.1, dtype=BF16, splits=0, ws=P, wsb=1 << 30)
    a.update(kw)
    return mha.mha_fwd_paged_validate(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["o"], a["lse"], a["B"],
                                      a["H"], a["Nq"], a["d"], a["nb"], a["bs"], a["mb"], a["scale"],
                                      a["dtype"], a["splits"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(dtype=F32, d=64, bs=256), OK), (dict(dtype=F16, splits=3, bs=65536, mb=16), OK),
    (dict(bt=P + 4, sl=P + 12), OK), (dict(bs=32, Nq=7), OK),
    (dict(bt=0), INVALID), (dict(sl=0), INVALID), (dict(kp=0), INVALID), (dict(ws=0), INVALID),
    (dict(wsb=16), INVALID), (dict(nb=0), INVALID), (dict(mb=0), INVALID), (dict(Nq=0), INVALID),
    (dict(splits=-1), INVALID), (dict(dtype=5), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(bs=8), UNSUPPORTED), (dict(bs=48), UNSUPPORTED), (dict(bs=131072), UNSUPPORTED),
    (dict(d=32), UNSUPPORTED), (dict(bt=P + 2), UNSUPPORTED), (dict(sl=P + 1), UNSUPPORTED),
    (dict(vp=P + 8), UNSUPPORTED), (dict(bs=65536, mb=1 << 15), UNSUPPORTED),
])
def test_paged_validate(kw, code):
    assert pv(**kw) == code


def test_paged_rejects_before_launch():
    assert mha.mha_fwd_paged(P, P, P, P, P, P, P, 1, 1, 1, 64, 10, 16, 4, 0.1, BF16, 0, 0, 0, 0) == INVALID
    assert mha.mha_fwd_paged(P, P, P, P, P, P, P, 1, 1, 1, 64, 10, 24, 4, 0.1, BF16, 0, P, 1 << 20, 0) \
        == UNSUPPORTED


@pytest.mark.parametrize("B,H,Nq,bs,mb", [(1, 1, 1, 16, 1), (64, 8, 1, 16, 512), (16, 32, 1, 64, 256),
                                          (8, 8, 1, 256, 128), (32, 16, 4, 32, 128), (2, 2, 200, 128, 3)])
@pytest.mark.parametrize("splits", [0, 1, 3, 10000])
def test_paged_partition(B, H, Nq, bs, mb, splits):
    max_keys = bs * mb
    s = mha.mha_fwd_paged_splits(B, H, Nq, bs, mb, splits)
    tiles = -(-max_keys // 64)
    assert 1 <= s <= tiles
    if splits > 0:
        assert s <= splits
    else:
        # the split-KV choice over the longest possible sequence
        assert s == mha.mha_fwd_splitkv_splits(B, H, Nq, max_keys, 0)
    assert mha.mha_fwd_paged_workspace_size(B, H, Nq, 128, bs, mb, splits) == s * B * H * Nq * 129 * 4
    assert mha.mha_fwd_paged_splits(B, H, Nq, 24, mb, splits) == 0
    assert mha.mha_fwd_paged_workspace_size(B, H, Nq, 128, bs, 0, splits) == 0


def test_paged_bytes():
    assert mha.mha_fwd_paged_bytes(64, 8, 1, 263473, 128, BF16) == \
        (2 * 64 + 2 * 263473) * 8 * 128 * 2 + 4 * 64 * 8
    assert mha.mha_fwd_paged_bytes(2, 3, 4, 5, 64, F32) == (2 * 2 * 4 + 2 * 5) * 3 * 64 * 4 + 4 * 2 * 3 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(dtype=F16), OK), (dict(M=1, N=8, K=8), OK),
    (dict(a=0), INVALID), (dict(c=0), INVALID), (dict(M=0), INVALID), (dict(K=-8), INVALID), (dict(dtype=7), INVALID),
    (dict(dtype=F32), UNSUPPORTED), (dict(N=12), UNSUPPORTED), (dict(K=100), UNSUPPORTED),
    (dict(b=P + 8), UNSUPPORTED), (dict(M=1 << 20, K=4096), UNSUPPORTED), (dict(N=1 << 19, K=8192), UNSUPPORTED),
    (dict(M=(1 << 27) - 1, N=(1 << 27) - 8, K=8), UNSUPPORTED),
])
def test_gemm_validate(kw, code):
    a = dict(a=P, b=P, c=P, M=1000, N=4096, K=4096, dtype=BF16)
    a.update(kw)
    assert mha.mha_gemm_validate(a["a"], a["b"], a["c"], a["M"], a["N"], a["K"], a["dtype"]) == code


def test_gemm_rejects_before_launch_and_accounting():
    assert mha.mha_gemm(P, P, 0, 8, 8, 8, BF16, 0) == INVALID
    assert mha.mha_gemm_flops(1024, 4096, 14336) == 2.0 * 1024 * 4096 * 14336
    assert mha.mha_gemm_bytes(1024, 4096, 14336, BF16) == (1024 * 14336 + 14336 * 4096 + 1024 * 4096) * 2


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(splits=3), OK), (dict(dtype=F16, M=1, N=8, K=8), OK),
    (dict(ws=0), INVALID), (dict(wsb=16), INVALID), (dict(splits=-2), INVALID), (dict(a=0), INVALID),
    (dict(ws=P + 4), UNSUPPORTED), (dict(K=12), UNSUPPORTED), (dict(dtype=F32), UNSUPPORTED),
])
def test_gemm_splitk_validate(kw, code):
    a = dict(a=P, b=P, c=P, M=16, N=4096, K=14336, dtype=BF16, splits=0, ws=P, wsb=1 << 30)
    a.update(kw)
    assert mha.mha_gemm_splitk_validate(a["a"], a["b"], a["c"], a["M"], a["N"], a["K"], a["dtype"], a["splits"],
                                        a["ws"], a["wsb"]) == code


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (16, 14336, 4096), (16, 4096, 14336), (65536, 64, 4096),
                                   (300, 520, 200), (128, 128, 65536), (16, 1000, 4104)])
@pytest.mark.parametrize("splits", [0, 1, 3, 100000])
def test_gemm_splitk_partition(M, N, K, splits):
    s = mha.mha_gemm_splitk_splits(M, N, K, splits)
    steps = -(-K // 64)
    assert 1 <= s <= steps
    if splits > 0:
        assert s <= splits
    else:
        tiles = -(-M // 128) * -(-N // 128)
        want = min(-(-512 // tiles), (steps + 3) // 4)
        p2 = 1
        while p2 * 2 <= want:
            p2 *= 2
        assert s == -(-steps // -(-steps // p2))       # ranges of ceil(steps / p2) steps
    assert mha.mha_gemm_splitk_workspace_size(M, N, K, splits) == s * M * N * 4
    assert mha.mha_gemm_splitk(P, P, P, M, N, K, BF16, splits, 0, 0, 0) == INVALID
