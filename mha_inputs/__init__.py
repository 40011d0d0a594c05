"""Seeded synthetic inputs for multi-head attention forward.

This module is the only code shared by the oracle side and the GPU side. It draws
random numbers and encodes them; it contains none of the attention arithmetic.

Draw recipe (one reading, since the workloads only say "i.i.d. from seed"):
  * ``numpy.random.Generator(PCG64)`` seeded from ``SeedSequence(seed).spawn(3)``,
    one child stream each for Q, K and V, drawn in that order;
  * values are drawn in float32 (normal: ``standard_normal * sigma``; uniform:
    ``uniform(lo, hi)``), then, for bfloat16 or float16 workloads, encoded by
    round-to-nearest-even on the host;
  * the identical encoded bytes go to the GPU and to the oracle, which decodes
    them exactly.

Arrays are contiguous ``[B, H, N, d]``.  bf16 and fp16 tensors are returned as
``uint16`` bit patterns, fp32 tensors as ``float32``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "SWEEP",
    "DECODE",
    "PagedWorkload",
    "PAGED",
    "GemmWorkload",
    "GEMM",
    "GEMM_MEMBOUND",
    "draw_gemm",
    "f32_to_bf16_bits",
    "f32_to_f16_bits",
    "draw",
    "draw_qkv",
    "draw_paged",
    "draw_paged_workload",
    "paged_lengths",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values to bfloat16 bit patterns, round-to-nearest-even.

    Non-finite inputs are not expected (the draws are finite).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values to IEEE float16 bit patterns, round-to-nearest-even
    (numpy's float32 -> float16 conversion; values beyond 65504 round to inf)."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


@dataclass(frozen=True)
class Dist:
    """A value distribution: ``("normal", sigma)`` or ``("uniform", lo, hi)``."""

    kind: str
    a: float = 1.0
    b: float = 0.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32", "bf16" or "f16"
    causal: bool
    seed: int
    qk_dist: Dist = field(default_factory=lambda: Dist("normal", 1.0))
    v_dist: Dist = field(default_factory=lambda: Dist("normal", 1.0))
    Nk: int = 0   # keys per head when it differs from the N query rows (split-KV decoding)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.H, self.N, self.d)

    @property
    def kv_len(self) -> int:
        return self.Nk or self.N

    @property
    def kv_shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.H, self.kv_len, self.d)

    def credited_flops(self) -> float:
        """4*B*H*N*Nk*d, halved for the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.kv_len * self.d
        return f / 2.0 if self.causal else f


# The five attention-forward workloads: shapes, dtypes, distributions, masks.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("fp32_B1_H2_N128_d64", 1, 2, 128, 64, "f32", False, seed=1),
        Workload("bf16_B4_H16_N1024_d64", 4, 16, 1024, 64, "bf16", False, seed=2),
        Workload("bf16_B4_H32_N4096_d128_causal", 4, 32, 4096, 128, "bf16", True, seed=3),
        Workload("bf16_B1_H32_N16384_d128_causal", 1, 32, 16384, 128, "bf16", True, seed=4),
        Workload(
            "bf16_B8_H16_N8192_d64_stress",
            8, 16, 8192, 64, "bf16", False, seed=5,
            qk_dist=Dist("normal", 3.0),
            v_dist=Dist("uniform", -1.0, 1.0),
        ),
    ]
}


# The FlashAttention-2 forward sweep of the ML-Triton paper (section 4.2, Figures 13
# and 14): 32k tokens in total, sequence length 1k..32k, hidden size 2048 with head
# dimension 64 (32 heads) or 128 (16 heads); batch = 32768 / N.  The pages state neither
# the mask nor the value distribution: both masks are listed, with N(0,1) inputs, in
# the float16 of the pages' listings.
SWEEP: Dict[str, Workload] = {}
for _i, (_d, _causal, _N) in enumerate(
        (d, c, n) for d in (64, 128) for c in (False, True)
        for n in (1024, 2048, 4096, 8192, 16384, 32768)):
    _w = Workload(f"f16_T32k_N{_N}_d{_d}{'_causal' if _causal else ''}", 32768 // _N, 2048 // _d,
                  _N, _d, "f16", _causal, seed=100 + _i)
    SWEEP[_w.name] = _w


# Split-KV decoding: few query rows against a long key/value sequence, no mask.  The
# pages give no sizes (only that the query length is typically 1): batch x heads x keys
# are chosen to stream 0.5-1 GiB of K/V per call.
DECODE: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("bf16_decode_B8_H8_Nk32768_d128", 8, 8, 1, 128, "bf16", False, seed=200, Nk=32768),
        Workload("bf16_decode_B64_H8_Nk4096_d128", 64, 8, 1, 128, "bf16", False, seed=201, Nk=4096),
        Workload("bf16_decode_B8_H8_Nk32768_d128_q4", 8, 8, 4, 128, "bf16", False, seed=202, Nk=32768),
        Workload("bf16_decode_B1_H8_Nk131072_d128", 1, 8, 1, 128, "bf16", False, seed=203, Nk=131072),
        Workload("f16_decode_B16_H16_Nk8192_d64", 16, 16, 1, 64, "f16", False, seed=204, Nk=8192),
    ]
}


@dataclass(frozen=True)
class PagedWorkload:
    """Decoding against a paged key/value cache.

    ``B`` sequences of ``H`` heads, ``Nq`` query rows each; sequence lengths drawn
    uniformly from ``[len_lo, len_hi]`` (or all equal when ``len_lo == len_hi``);
    blocks of ``block_size`` keys; the pool holds the used blocks plus ``spare``
    unused ones.  See :func:`draw_paged`.
    """

    name: str
    B: int
    H: int
    Nq: int
    d: int
    dtype: str
    block_size: int
    len_lo: int
    len_hi: int
    seed: int
    spare: int = 16

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


# Paged decoding.  The pages give neither sizes nor a block size: a serving-style mix of
# sequence lengths with the small blocks of paged KV caches (16 keys), a long-context
# case with large blocks, the contiguous split-KV decoding shape with 256-key blocks (the
# cost of the indirection), and an fp16 d=64 case with several query rows.
PAGED: Dict[str, PagedWorkload] = {
    w.name: w
    for w in [
        PagedWorkload("bf16_paged_B64_H8_d128_bs16_len512-8192", 64, 8, 1, 128, "bf16", 16, 512, 8192, seed=300),
        PagedWorkload("bf16_paged_B16_H32_d128_bs64_len1024-16384", 16, 32, 1, 128, "bf16", 64, 1024, 16384,
                      seed=301),
        PagedWorkload("bf16_paged_B8_H8_d128_bs256_len32768", 8, 8, 1, 128, "bf16", 256, 32768, 32768, seed=302),
        PagedWorkload("f16_paged_B32_H16_d64_bs32_q4_len256-4096", 32, 16, 4, 64, "f16", 32, 256, 4096, seed=303),
    ]
}


@dataclass(frozen=True)
class GemmWorkload:
    """C [M, N] = A [M, K] @ B [K, N], row-major, N(0,1) operands."""

    name: str
    M: int
    N: int
    K: int
    dtype: str
    seed: int

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


# Dense GEMM (the tiled contraction of the ML-Triton paper, sections 2 and 4.1).  The
# pages keep only "m = 1k..16k, shapes from Llama-2 / Llama-3 layers": the token count
# M runs over 1k..16k against three Llama-3-8B linear layers (hidden 4096, MLP 14336):
# the attention output projection (K = N = 4096), the MLP up projection (K = 4096,
# N = 14336) and the MLP down projection (K = 14336, N = 4096).
GEMM: Dict[str, GemmWorkload] = {}
for _i, ((_k, _n), _m) in enumerate(((kn, m) for kn in ((4096, 4096), (4096, 14336), (14336, 4096))
                                     for m in (1024, 2048, 4096, 8192, 16384))):
    _g = GemmWorkload(f"bf16_gemm_M{_m}_N{_n}_K{_k}", _m, _n, _k, "bf16", seed=400 + _i)
    GEMM[_g.name] = _g


# Memory-bound GEMMs (section 4.1, Figure 12): the pages keep "large m, large k and large
# n" and the next-token stage.  One large dimension at a time against Llama-3-8B sizes:
# a 64-way router over 64k tokens (large M), and 16 decoding tokens through the MLP up
# (large N) and down (large K) projections.
GEMM_MEMBOUND: Dict[str, GemmWorkload] = {
    g.name: g
    for g in [
        GemmWorkload("bf16_gemm_M65536_N64_K4096", 65536, 64, 4096, "bf16", seed=450),
        GemmWorkload("bf16_gemm_M16_N14336_K4096", 16, 14336, 4096, "bf16", seed=451),
        GemmWorkload("bf16_gemm_M16_N4096_K14336", 16, 4096, 14336, "bf16", seed=452),
    ]
}


def _sample(rng: np.random.Generator, shape, dist: Dist) -> np.ndarray:
    if dist.kind == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if dist.a != 1.0:
            x *= np.float32(dist.a)
        return x
    if dist.kind == "uniform":
        return rng.uniform(dist.a, dist.b, size=shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist.kind!r}")


def draw(shape, dtype: str, seed: int, qk_dist: Dist = Dist("normal", 1.0),
         v_dist: Dist = Dist("normal", 1.0), kv_shape=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Draw Q of ``shape`` (``[B,H,N,d]``) and K, V of ``kv_shape`` (default ``shape``)
    from ``seed``.

    Returns float32 arrays for ``dtype == "f32"`` and uint16 bit patterns for
    ``dtype == "bf16"`` or ``"f16"``.
    """
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    children = np.random.SeedSequence(seed).spawn(3)
    out = []
    shapes = (shape, kv_shape or shape, kv_shape or shape)
    for child, dist, shp in zip(children, (qk_dist, qk_dist, v_dist), shapes):
        rng = np.random.Generator(np.random.PCG64(child))
        x = _sample(rng, shp, dist)
        if dtype == "bf16":
            x = f32_to_bf16_bits(x)
        elif dtype == "f16":
            x = f32_to_f16_bits(x)
        out.append(np.ascontiguousarray(x))
    return out[0], out[1], out[2]


def draw_qkv(w: Workload):
    """Q, K, V for one of the named workloads."""
    return draw(w.shape, w.dtype, w.seed, w.qk_dist, w.v_dist, w.kv_shape if w.Nk else None)


def draw_paged(B: int, H: int, Nq: int, d: int, dtype: str, block_size: int, seq_lens, seed: int,
               spare: int = 16, dist: Dist = Dist("normal", 1.0)):
    """Q and a paged K/V cache from ``seed``.

    ``seq_lens``: ``B`` key counts.  Every sequence gets ``ceil(len / block_size)``
    physical blocks; the pool holds those plus ``spare`` more, and the physical block
    ids are a seeded random permutation, so the blocks of one sequence are scattered
    over the pool.  Table entries past a sequence's last block are -1.  Returns
    ``(q [B,H,Nq,d], k_pool, v_pool [num_blocks,H,block_size,d], block_table
    [B, max_blocks] int32, seq_lens [B] int32)``, values encoded as for :func:`draw`
    (the unused rows of the pool hold draws too).
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.shape != (B,) or (lens < 0).any():
        raise ValueError("need B non-negative sequence lengths")
    per_seq = (lens + block_size - 1) // block_size
    max_blocks = max(1, int(per_seq.max()))
    num_blocks = int(per_seq.sum()) + int(spare)
    if num_blocks < 1:
        raise ValueError("empty pool")
    children = np.random.SeedSequence(seed).spawn(4)
    perm = np.random.Generator(np.random.PCG64(children[0])).permutation(num_blocks)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        n = int(per_seq[b])
        table[b, :n] = perm[at:at + n]
        at += n
    pool_shape = (num_blocks, H, block_size, d)
    q, k, v = draw((B, H, Nq, d), dtype, int(children[1].generate_state(1)[0]), dist, dist, kv_shape=pool_shape)
    return q, k, v, table, lens.astype(np.int32)


def paged_lengths(w: PagedWorkload) -> np.ndarray:
    """The sequence lengths of a paged workload (seeded, uniform in [len_lo, len_hi])."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed).spawn(1)[0]))
    return rng.integers(w.len_lo, w.len_hi + 1, size=w.B).astype(np.int64)


def draw_paged_workload(w: PagedWorkload):
    """Inputs of a named paged workload (see :func:`draw_paged`)."""
    return draw_paged(w.B, w.H, w.Nq, w.d, w.dtype, w.block_size, paged_lengths(w), w.seed + 1, w.spare)


def draw_gemm(M: int, N: int, K: int, dtype: str, seed: int, dist: Dist = Dist("normal", 1.0)):
    """A ``[M, K]`` and B ``[K, N]`` from ``seed`` (two child streams), encoded as for
    :func:`draw`."""
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    out = []
    for child, shp in zip(np.random.SeedSequence(seed).spawn(2), ((M, K), (K, N))):
        x = _sample(np.random.Generator(np.random.PCG64(child)), shp, dist)
        if dtype == "bf16":
            x = f32_to_bf16_bits(x)
        elif dtype == "f16":
            x = f32_to_f16_bits(x)
        out.append(np.ascontiguousarray(x))
    return out[0], out[1]
