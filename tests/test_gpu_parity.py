"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on identical
seeded inputs.  Tolerances: fp32 inputs max|dO|, max|dLSE| <= 1e-4; bf16 inputs
max|dO| <= 2e-2, max|dLSE| <= 1e-3; fp16 inputs max|dO| <= 5e-3, max|dLSE| <= 1e-3."""
import math

import numpy as np
import pytest
import torch

import head_attention_fa2_amd as mha
import mha_inputs
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

W = mha_inputs.WORKLOADS


def _check(o, lse, o_ref, l_ref, dtype, what, magnitude=1.0, magnitude_lse=None):
    tol_o, tol_l = gu.TOL[dtype]
    tol_o, tol_l = tol_o * magnitude, tol_l * (magnitude if magnitude_lse is None else magnitude_lse)
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse - l_ref)))
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    assert eo <= tol_o, f"{what}: O error {eo}"
    assert el <= tol_l, f"{what}: LSE error {el}"


# ---------------------------------------------------------------- element-wise, small
# Each workload at a size the oracle evaluates whole in seconds: several 128-row query
# blocks and 64-key tiles, with ragged tails where N is not a multiple of them.
SMALL = [
    ("fp32_B1_H2_N128_d64", dict(B=1, H=2, N=128)),                  # the full workload
    ("bf16_B4_H16_N1024_d64", dict(B=4, H=16, N=1024)),              # the full workload
    ("bf16_B4_H32_N4096_d128_causal", dict(B=2, H=3, N=1000)),
    ("bf16_B1_H32_N16384_d128_causal", dict(B=1, H=2, N=2049)),
    ("bf16_B8_H16_N8192_d64_stress", dict(B=2, H=2, N=1100)),
]


# fp16 inputs (the element type of the pages' listings), several tiles and ragged tails
SMALL_F16 = [(1, 2, 1000, 128, True), (2, 3, 777, 64, False), (1, 4, 1100, 128, False), (2, 2, 300, 64, True)]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL_F16)
def test_f16_elementwise(B, H, N, d, causal):
    q, k, v = gu.draw(B, H, N, d, "f16", seed=500 + N + d)
    scale = 1 / math.sqrt(d)
    o, lse = gu.run(q, k, v, "f16", causal, scale)
    o_ref, l_ref = gu.oracle_full(q, k, v, "f16", causal, scale)
    _check(o, lse, o_ref, l_ref, "f16", f"f16 B{B} H{H} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
def test_workload_elementwise(name, shape):
    w = W[name]
    q, k, v = mha_inputs.draw((shape["B"], shape["H"], shape["N"], w.d), w.dtype, w.seed,
                              w.qk_dist, w.v_dist)
    o, lse = gu.run(q, k, v, w.dtype, w.causal, w.scale)
    o_ref, l_ref = gu.oracle_full(q, k, v, w.dtype, w.causal, w.scale)
    _check(o, lse, o_ref, l_ref, w.dtype, f"{name} {shape}")


# ---------------------------------------------------------------- full size, every element
@pytest.mark.parametrize("name", [n for n in W if n not in ("fp32_B1_H2_N128_d64", "bf16_B4_H16_N1024_d64")])
def test_workload_full_size_elementwise(name):
    """The full workload in the launch configuration the benchmark times, compared with
    the float64 oracle on EVERY output element (O and LSE); also every output finite and
    within the convex-combination bound |O| <= max|V|.  (The two smaller workloads are
    compared whole by test_workload_elementwise.)"""
    w = W[name]
    q, k, v = mha_inputs.draw_qkv(w)
    print(f"{name}: launching the full workload", flush=True)
    tq, tk, tv = (gu.to_device(x, w.dtype) for x in (q, k, v))
    o, lse = mha.fwd(tq, tk, tv, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    vmax = float(tv.float().abs().amax())
    assert float(o.float().abs().amax()) <= vmax * (1 + 2 ** -7) + 1e-6
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    del tq, tk, tv, o, lse
    print(f"{name}: oracle on {gu.host_threads()} threads", flush=True)
    o_ref, l_ref = gu.oracle_full(q, k, v, w.dtype, w.causal, w.scale, threads=gu.host_threads())
    _check(og, lg, o_ref, l_ref, w.dtype, f"{name} full, all {og.shape[0] * og.shape[1] * og.shape[2]} rows")


# ---------------------------------------------------------------- edge cases
EDGE = []
for dtype in ("bf16", "f32", "f16"):
    for d in (64, 128):
        for N in (1, 2, 63, 64, 65, 127, 129, 200, 257):
            for causal in (False, True):
                EDGE.append((1, 1, N, d, causal, dtype))
EDGE += [(3, 5, 130, 64, True, "bf16"), (2, 1, 513, 128, False, "bf16"), (1, 3, 300, 64, True, "f32")]


@pytest.mark.parametrize("B,H,N,d,causal,dtype", EDGE)
def test_edge_shapes(B, H, N, d, causal, dtype):
    q, k, v = gu.draw(B, H, N, d, dtype, seed=1000 + N + d, qk_sigma=1.5)
    scale = 1 / math.sqrt(d)
    o, lse = gu.run(q, k, v, dtype, causal, scale)
    o_ref, l_ref = gu.oracle_full(q, k, v, dtype, causal, scale)
    _check(o, lse, o_ref, l_ref, dtype, f"edge B{B} H{H} N{N} d{d} causal={causal} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_scales_and_large_logits(dtype):
    B, H, N, d = 1, 2, 300, 64
    for sigma, scale in ((3.0, 0.125), (1.0, 1.0), (1.0, -0.3), (5.0, 0.5), (1.0, 0.0)):
        q, k, v = gu.draw(B, H, N, d, dtype, seed=int(sigma * 10), qk_sigma=sigma)
        for causal in (False, True):
            o, lse = gu.run(q, k, v, dtype, causal, scale)
            o_ref, l_ref = gu.oracle_full(q, k, v, dtype, causal, scale)
            # fp32 logits of size |s| carry rounding of order |s| * 2^-24 * sqrt(d) from the
            # float32 dot product itself; past |lse| ~ 16 the absolute bound scales with it.
            mag = max(1.0, float(np.max(np.abs(l_ref))) / 16.0) if dtype == "f32" else 1.0
            _check(o, lse, o_ref, l_ref, dtype, f"sigma={sigma} scale={scale} causal={causal}", mag)


# Seeded random shapes (both kernel forms, every element type, ragged N, both masks),
# element-wise against the oracle.
def _random_cases(n=24, seed=9001):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.45, 0.35, 0.2]))
        N = int(rng.integers(1, 700))
        heads = int(rng.integers(1, 400 if N < 200 else (120 if N < 450 else 60)))
        B = int(rng.integers(1, 4))
        cases.append((B, max(1, heads // B), N, d, bool(rng.integers(0, 2)), dtype, float(rng.choice([1.0, 2.0]))))
    return cases


@pytest.mark.parametrize("B,H,N,d,causal,dtype,sigma", _random_cases())
def test_random_shapes_elementwise(B, H, N, d, causal, dtype, sigma):
    q, k, v = gu.draw(B, H, N, d, dtype, seed=8000 + B * 1000 + H * 10 + N, qk_sigma=sigma)
    scale = 1 / math.sqrt(d)
    o, lse = gu.run(q, k, v, dtype, causal, scale)
    o_ref, l_ref = gu.oracle_full(q, k, v, dtype, causal, scale, threads=gu.host_threads())
    # O of 16-bit inputs: rounding P and then O to the element type (round to nearest,
    # unit roundoff u = 2^-8 for bf16, 2^-11 for fp16) costs at most 2 u max|V|.  The flat
    # tolerances hold the benchmark draws with room to spare; these draws (peaky rows at
    # sigma = 2, millions of N(0,1) values of V) are held to that bound when it is wider.
    # fp32: the logit reading of test_scales_and_large_logits.  The LSE bound stays flat.
    vmax = float(np.max(np.abs(oracle.decode(v, dtype))))
    if dtype == "f32":
        mag = max(1.0, float(np.max(np.abs(l_ref))) / 16.0)
        mag_l = mag
    else:
        bound = 2.0 * (2.0 ** -8 if dtype == "bf16" else 2.0 ** -11) * vmax
        mag = max(1.0, bound / gu.TOL[dtype][0])
        mag_l = 1.0
    _check(o, lse, o_ref, l_ref, dtype, f"random B{B} H{H} N{N} d{d} causal={causal} {dtype} sigma={sigma}", mag,
           mag_l)


# Rows whose maximum keeps climbing: key norms ramp up along the sequence, Q has a
# positive mean, and a few keys are spikes along that mean, so that some logits jump far
# above every earlier one (up to ~200, where exp of the old offset overflows float32).
# The kernel's exponent offset must move on such tiles (the scores re-formed, the row
# max taken, O and l rescaled); in both kernel forms (small and large grids).
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 2, 700), (1, 90, 300)])
def test_offset_moves_elementwise(dtype, d, B, H, N):
    rng = np.random.default_rng(7000 + d + N)
    q = rng.standard_normal((B, H, N, d)).astype(np.float32) + 0.5
    k = rng.standard_normal((B, H, N, d)).astype(np.float32)
    k *= (1.0 + 3.0 * np.arange(N) / N).astype(np.float32)[None, None, :, None]
    scale = 1 / math.sqrt(d)
    for j, logit in ((N // 5, 20.0), (N // 3, 60.0), (2 * N // 3, 200.0), (N - 1, 30.0)):
        k[:, :, j, :] = logit / (0.5 * d * scale)      # q.k * scale ~ logit on average
    v = rng.uniform(-1.0, 1.0, (B, H, N, d)).astype(np.float32)
    enc = {"bf16": mha_inputs.f32_to_bf16_bits, "f16": mha_inputs.f32_to_f16_bits, "f32": lambda a: a}[dtype]
    q, k, v = enc(q), enc(k), enc(v)
    for causal in (False, True):
        o, lse = gu.run(q, k, v, dtype, causal, scale)
        o_ref, l_ref = gu.oracle_full(q, k, v, dtype, causal, scale)
        mag = max(1.0, float(np.max(np.abs(l_ref))) / 16.0) if dtype == "f32" else 1.0
        _check(o, lse, o_ref, l_ref, dtype, f"offset moves {dtype} d{d} B{B} H{H} N{N} causal={causal}", mag)


# ---------------------------------------------------------------- invariants on GPU output
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_invariants_on_gpu(dtype, d):
    B, H, N = 1, 2, 333
    tol_o, tol_l = gu.TOL[dtype]
    q, k, v = gu.draw(B, H, N, d, dtype, seed=5)
    enc = {"bf16": mha_inputs.f32_to_bf16_bits, "f16": mha_inputs.f32_to_f16_bits,
           "f32": lambda x: x}[dtype]
    ones = enc(np.ones(v.shape, dtype=np.float32))
    zeros = np.zeros_like(q)
    vf = oracle.decode(v, dtype)
    for causal in (False, True):
        o1, _ = gu.run(q, k, ones, dtype, causal)
        assert np.max(np.abs(o1 - 1.0)) <= tol_o, "V = 1 gives O = 1"
        oz, lz = gu.run(zeros, k, v, dtype, causal)
        cnt = np.arange(1, N + 1, dtype=np.float64)
        mean = np.cumsum(vf, axis=2) / cnt[None, None, :, None] if causal else \
            np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
        lz_ref = np.log(cnt)[None, None] if causal else np.full(lz.shape, math.log(N))
        assert np.max(np.abs(oz - mean)) <= tol_o, "Q = 0 gives the mean of visible V"
        assert np.max(np.abs(lz - lz_ref)) <= tol_l, "Q = 0 gives lse = ln(#visible)"
    perm = np.random.default_rng(3).permutation(N)
    o, l = gu.run(q, k, v, dtype, False)
    op, lp = gu.run(q, k[:, :, perm].copy(), v[:, :, perm].copy(), dtype, False)
    assert np.max(np.abs(op - o)) <= tol_o and np.max(np.abs(lp - l)) <= tol_l, "key permutation"


# ---------------------------------------------------------------- determinism, streams, errors
def test_bitwise_repeatable_and_stream():
    w = W["bf16_B4_H32_N4096_d128_causal"]
    q, k, v = gu.draw(2, 4, 1500, 128, "bf16", seed=11)
    tq, tk, tv = (gu.to_device(x, "bf16") for x in (q, k, v))
    o1, l1 = mha.fwd(tq, tk, tv, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())      # inputs were written on the current stream
    with torch.cuda.stream(s):
        o2, l2 = mha.fwd(tq, tk, tv, causal=True)
    o3, l3 = mha.fwd(tq, tk, tv, causal=True, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)
    assert w.d == 128


def test_out_buffers_fully_overwritten():
    q, k, v = gu.draw(1, 2, 130, 64, "bf16", seed=12)
    tq, tk, tv = (gu.to_device(x, "bf16") for x in (q, k, v))
    out = torch.full_like(tq, float("nan"))
    lse = torch.full((1, 2, 130), float("nan"), device=tq.device)
    mha.fwd(tq, tk, tv, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())


# Causal launches with B*H a multiple of 8 take the grouped dispatch order (each XCD owns
# B*H/8 whole heads, run in groups of four, heaviest query blocks of a group first).
# Element-wise against the oracle with 1, 2, 3, 5, 9, 16 and 17 heads per XCD (one
# partial group for 3; a full group and a partial one for 5; two full groups and a
# partial one for 9; four full groups for 16, four and a partial one for 17) and ragged
# query blocks.
GROUPED = [(1, 8, 300, 64, "bf16"), (2, 8, 260, 128, "bf16"), (3, 8, 200, 64, "f16"),
           (5, 8, 257, 128, "bf16"), (1, 72, 130, 128, "f16"), (1, 8, 100, 128, "bf16"), (2, 4, 1, 64, "f16"),
           (2, 64, 140, 64, "bf16"), (1, 136, 129, 128, "f16"), (1, 264, 130, 64, "bf16")]


@pytest.mark.parametrize("B,H,N,d,dtype", GROUPED)
def test_causal_grouped_order_elementwise(B, H, N, d, dtype):
    q, k, v = gu.draw(B, H, N, d, dtype, seed=2000 + B * H + N)
    scale = 1 / math.sqrt(d)
    o, lse = gu.run(q, k, v, dtype, True, scale)
    o_ref, l_ref = gu.oracle_full(q, k, v, dtype, True, scale)
    _check(o, lse, o_ref, l_ref, dtype, f"grouped causal B{B} H{H} N{N} d{d} {dtype}")


# 16-bit launches of at most 256 workgroups with more than one K/V tile run the key-half
# form (8 wavefronts per workgroup, two halves of the key tiles merged at the end); larger
# grids the 4-wavefront form.  Shapes on both sides of the threshold, causal and not,
# with ragged query blocks.
FORMS = [(1, 128, 256, 64, False, "bf16"), (1, 130, 256, 64, False, "bf16"),      # 256 | 260 workgroups
         (1, 128, 256, 128, False, "f16"), (1, 130, 256, 128, False, "f16"),      # 256 | 260
         (1, 64, 500, 64, True, "bf16"), (1, 66, 500, 64, True, "bf16"),          # 256 | 264
         (1, 64, 510, 128, True, "bf16"), (1, 66, 510, 128, True, "f16"),         # 256 | 264
         (1, 4, 65, 128, True, "bf16"), (3, 5, 33, 128, False, "bf16"),           # two tiles / ragged
         (2, 3, 64, 64, False, "f16"), (2, 3, 65, 64, False, "f16")]              # one tile | two


@pytest.mark.parametrize("B,H,N,d,causal,dtype", FORMS)
def test_both_kernel_forms_elementwise(B, H, N, d, causal, dtype):
    q, k, v = gu.draw(B, H, N, d, dtype, seed=4000 + B * H + N + d)
    scale = 1 / math.sqrt(d)
    o, lse = gu.run(q, k, v, dtype, causal, scale)
    o_ref, l_ref = gu.oracle_full(q, k, v, dtype, causal, scale)
    _check(o, lse, o_ref, l_ref, dtype, f"forms B{B} H{H} N{N} d{d} causal={causal} {dtype}")


@pytest.mark.parametrize("B,H,N,d", [(4, 32, 4096, 128), (1, 32, 16384, 128), (3, 40, 1000, 64)])
def test_causal_every_row_written(B, H, N, d):
    """Full-size causal launches: outputs pre-filled with NaN come back finite, so every
    (head, query block) pair was taken by exactly one workgroup's dispatch slot."""
    g = torch.Generator(device="cuda").manual_seed(B * H + N)
    q, k, v = (torch.randn(B, H, N, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=q.device)
    mha.fwd(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("bf16", 64, False), ("f16", 128, False),
                                            ("f16", 64, True)])
def test_long_sequence_sampled(dtype, d, causal):
    """One head per batch entry with N = 65536 (2048 key tiles for the last query block):
    sampled rows, including the first and last of several query blocks, against the oracle."""
    B, H, N = 1, 2, 65536
    q, k, v = gu.draw(B, H, N, d, dtype, seed=4000 + d + int(causal))
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (gu.to_device(x, dtype) for x in (q, k, v))
    o, lse = mha.fwd(tq, tk, tv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rows = [0, 1, 127, 128, 4095, 32768, 65407, 65408, N - 1]
    picks = [(0, h, r) for h in range(H) for r in rows]
    o_ref, l_ref = oracle.attention_rows(q, k, v, causal=causal, scale=scale, picks=picks, dtype=dtype)
    idx = torch.tensor(picks, dtype=torch.long, device=o.device)
    og = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy().astype(np.float64)
    lg = lse[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy().astype(np.float64)
    _check(og, lg, o_ref, l_ref, dtype, f"long N={N} d{d} causal={causal} {dtype}")


def test_errors_raise():
    q = torch.zeros(1, 1, 16, 96, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(mha.MhaError) as e:
        mha.fwd(q, q, q)
    assert e.value.status == mha.MHA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        mha.fwd(q.double(), q.double(), q.double())
    with pytest.raises(ValueError):
        mha.fwd(q, q.float(), q)
