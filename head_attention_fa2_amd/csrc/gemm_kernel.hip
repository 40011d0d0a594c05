// Dense GEMM for gfx950 (AMD Instinct MI355X, CDNA4): C = A.B with A [M, K] and
// B [K, N] row-major in bf16 or fp16, float32 accumulation, C [M, N] rounded to the
// input type (round to nearest even).
//
// This is the tiled contraction of "ML-Triton, A Multi-Level Compilation and Language
// Extension to Triton GPU Programming", section 2 (a workgroup owns a block of C and
// accumulates it over k-steps, then stores it once; section 4.1 measures it on
// compute-bound LLM shapes), laid out for CDNA4:
//  * A workgroup of 8 wavefronts owns a 256 x 256 block of C; the wavefronts form a
//    2 x 4 grid and each accumulates a 128 x 64 sub-block in 8 float32 accumulators of
//    v_mfma_f32_32x32x16_{bf16,f16} (128 VGPRs).  One workgroup per CU (128 KiB of LDS).
//    Grids of fewer than 192 such tiles use 128 x 128 blocks of 4 wavefronts (64 x 64
//    each, two workgroups per CU) instead, and grids of fewer than 384 of those 128 x 64
//    blocks (64 x 32 per wavefront, three workgroups per CU), so that they fill the CUs.
//  * The product is formed transposed per 32 x 32 block, C^T = B^T.A^T, so that after
//    the MFMA every lane holds 8 consecutive columns of one row of C (16-byte stores).
//    The B^T operand comes from row-major B in LDS through ds_read_b64_tr_b16, the
//    A^T operand from row-major A through ds_read_b128; the rows of B^T enter in an
//    order that swaps bits 2 and 3 of the row index, which is what puts 8 consecutive
//    columns in one lane.
//  * k-steps of 64: the A (256 x 64) and B (64 x 256) tiles are copied HBM -> LDS with
//    global_load_lds_dwordx4, double buffered with one barrier per k-step (the copy of
//    step t+1 is in flight while step t is consumed; its A and B parts are issued after
//    the first and the second 16-wide substep of step t).  LDS rows are XOR-swizzled in
//    16-byte chunks so that both operand reads are free of bank conflicts.
//  * Workgroup ids are renumbered so that each XCD gets a contiguous range of tiles,
//    traversed in groups of 8 block-rows (the grouped order of the Triton tutorial's
//    GEMM), so the workgroups resident on one XCD share A and B panels in its L2.
//  * Ragged M and N: out-of-range rows / columns of A and B are read clamped and never
//    stored.  Ragged K (a multiple of 8): the A chunks past K are zeroed in LDS once
//    their copy has landed, so they add nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gfx950_lds.h"

// MHA_SERIALIZE=1: the race-check form of the k-step loop (one LDS buffer, each k-step
// copied, waited for and fenced by barriers before and after it is read); same
// arithmetic in the same order, so results equal the pipelined kernel's bit for bit.
#ifndef MHA_SERIALIZE
#define MHA_SERIALIZE 0
#endif
#include "mha_launch.h"
#include "mha_layout.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace mha_impl {
namespace {

using gfx950::copy_to_lds;
using gfx950::lds_addr;
using gfx950::tile_barrier;
using gfx950::wait_vmcnt;
using mha_layout::lds_inv;
using mha_layout::lds_off;
using mha_layout::v_operand_off;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

template <typename T>
struct Mfma;
template <>
struct Mfma<__bf16> {
  typedef bf16x8_t v8;
  static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma<_Float16> {
  typedef f16x8_t v8;
  static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Tile configurations: a workgroup owns a BM x BN block of C with WM x WN wavefronts,
// each accumulating (BM/WM) x (BN/WN) in 32 x 32 MFMA blocks; k-steps of 64.  KG > 1:
// KG groups of WM x WN wavefronts, each summing its own contiguous share of the k-steps
// through its own LDS stages; the groups' sums are added through LDS at the end (a split
// of K inside the workgroup: no workspace, C still rounded once).
template <int BM_, int BN_, int WM_, int WN_, int KG_ = 1>
struct Tiling {
  static constexpr int BM = BM_, BN = BN_, BK = 64, KG = KG_;
  static constexpr int WM = WM_, WN = WN_, Waves = WM * WN, Threads = 64 * Waves * KG;
  static constexpr int MB = BM / WM / 32, NB = BN / WN / 32;   // 32x32 blocks per wavefront
  static constexpr int RB = BN / 8;                           // 16-byte chunks per B row
  static constexpr int ATile = BM * BK * 2, BTile = BK * BN * 2, Stage = ATile + BTile;
  static constexpr int LoadsA = ATile / 16 / (64 * Waves), LoadsB = BTile / 16 / (64 * Waves);
  static_assert(LoadsA * 16 * 64 * Waves == ATile && LoadsB * 16 * 64 * Waves == BTile, "even split");
  static_assert(KG == 1 || 2 * Stage >= Waves * (BM / WM) * (BN / WN) * 4, "group sums fit its stages");
  static_assert(MB >= 1 && NB >= 1 && (RB == 8 || RB == 16 || RB == 32), "supported shapes");
};
// 256 x 256, 8 wavefronts of 128 x 64, one workgroup per CU (128 KiB of LDS).
typedef Tiling<256, 256, 2, 4> Large;
// 128 x 128, 4 wavefronts of 64 x 64, two workgroups per CU (64 KiB of LDS each): four
// times the tiles, for grids that would not fill the 256 CUs.
typedef Tiling<128, 128, 2, 2> Small;
// 128 x 64, 4 wavefronts of 64 x 32, three workgroups per CU (48 KiB of LDS each).
typedef Tiling<128, 64, 2, 2> Tiny;
// 128 x 128 with the k-steps split between two groups of 4 wavefronts of 64 x 64, one
// workgroup of 8 wavefronts per CU (2 x 64 KiB of LDS): the 128 x 128 blocks' operand
// reuse for grids too small to fill the CUs with 128 x 128 tiles.
typedef Tiling<128, 128, 2, 2, 2> Duo;
constexpr int kGroupM = 8;                 // block-rows per group of the tile order
// Below this many 256 x 256 tiles (3/4 of the 256 CUs) the 128 x 128 tiling is used.
// Measured on the Llama-3-8B shapes: 64 and 128 tiles run 1.2-1.7x faster as 128 x 128,
// 224 tiles and more 1.2-1.3x slower.
constexpr long kLargeMinTiles = 192;
// Below this many 128 x 128 tiles (1.5 per CU) the 128 x 64 tiling is used: measured
// 1.15-1.2x faster at 48-256 tiles, 1.5x slower at 512 ...
constexpr long kSmallMinTiles = 384;
// ... unless K is at least this long: then the 128 x 128 tiling with the k-steps split
// between two groups of wavefronts (measured at 256 tiles: 1.21x the 128 x 64 tiling at
// K = 4096 and 1.28x at K = 14336; at K = 1000 it was 0.85x).
constexpr int kDuoMinK = 2048;

struct GemmParams {
  const void* a;
  const void* b;
  void* c;
  int M, N, K;
  int tiles_m, tiles_n, total;   // total: tiles of C
  // split-K only: K per split (a multiple of the k-step), splits, float32 partial
  // products [splits][M][N]
  int kchunk = 0;
  int splits = 1;
  float* part = nullptr;
};

// SPLITK: workgroup (split, tile) sums k in [split*kchunk, min(K, (split+1)*kchunk))
// and stores its float32 partial block; gemm_splitk_reduce adds the partials.
template <typename T, typename C, bool SPLITK = false>
__global__ __launch_bounds__(C::Threads) void gemm_kernel(GemmParams p) {
  typedef typename Mfma<T>::v8 v8_t;
  constexpr int kBM = C::BM, kBN = C::BN, kBK = C::BK, kWaves = C::Waves, kWavesN = C::WN;
  constexpr int kMB = C::MB, kNB = C::NB, kATile = C::ATile, kStage = C::Stage;
  constexpr int kLoadsA = C::LoadsA, kLoadsB = C::LoadsB, kRB = C::RB, kKG = C::KG;
  static_assert(!(SPLITK && kKG > 1), "split-K over workgroups uses one k-group");
  __shared__ __attribute__((aligned(1024))) char lds[kKG * 2 * kStage];   // [group][buf][A, B]

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kgrp = wave_all / kWaves;             // k-group of this wavefront
  const int wave = wave_all - kgrp * kWaves;      // wavefront within its group
  char* const smem = lds + kgrp * 2 * kStage;     // this group's stages
  const int wave_m = wave / kWavesN, wave_n = wave % kWavesN;
  const int G = lane >> 5;

  // --- workgroup -> tile: contiguous id ranges per XCD, grouped block-row order.
  const int grid = SPLITK ? p.total * p.splits : p.total;
  int id = blockIdx.x;
  if ((grid & 7) == 0) id = (id & 7) * (grid >> 3) + (id >> 3);
  int kbeg = 0;
  if constexpr (SPLITK) {
    const int split = id / p.total;
    id -= split * p.total;
    kbeg = split * p.kchunk;
  }
  const int group = kGroupM * p.tiles_n;
  const int first_m = id / group * kGroupM;
  const int gsize = min(p.tiles_m - first_m, kGroupM);
  const int in_group = id % group;
  const int m0 = (first_m + in_group % gsize) * kBM;
  const int n0 = in_group / gsize * kBN;
  const int M = p.M, N = p.N, K = p.K;
  const unsigned lda = (unsigned)K * 2u, ldb = (unsigned)N * 2u;

  // --- tile loader.  Load j of a thread fills LDS slot (j*kWaves + wave)*64 + lane of
  // its tile; lds_inv gives the (row, chunk) that slot holds.  Byte offsets are 32-bit
  // (the host checks that A and B are under 4 GiB).
  unsigned a_row[kLoadsA];   // byte offset of the (clamped) A row
  int a_k[kLoadsA];          // k of the chunk within a tile
  int b_row[kLoadsB];        // k row within a tile
  unsigned b_col[kLoadsB];   // byte offset of the (clamped) column chunk
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    int r, c;
    lds_inv<8>((j * kWaves + wave) * 64 + lane, r, c);
    a_row[j] = (unsigned)min(m0 + r, M - 1) * lda;
    a_k[j] = c * 8;
  }
#pragma unroll
  for (int j = 0; j < kLoadsB; ++j) {
    int r, c;
    lds_inv<kRB>((j * kWaves + wave) * 64 + lane, r, c);
    b_row[j] = r;
    b_col[j] = (unsigned)min(n0 / 8 + c, N / 8 - 1) * 16u;
  }
  const int kend = SPLITK ? min(K, kbeg + p.kchunk) : K;
  int nk = (kend - kbeg + kBK - 1) / kBK;
  int nsteps = nk;               // steps of the workgroup's loop (every group's barriers)
  if constexpr (kKG > 1) {
    // k-steps [0, h) for group 0, [h, nk) for group 1
    const int h = (nk + 1) / 2;
    nsteps = h;
    if (kgrp == 1) {
      kbeg = h * kBK;
      nk -= h;
    } else {
      nk = h;
    }
  }

  // full k-steps: uniform (SGPR) bases advanced by k0 and per-lane offsets fixed for
  // the whole loop, so a copy costs no vector arithmetic
  unsigned a_off[kLoadsA], b_off[kLoadsB];
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) a_off[j] = a_row[j] + (unsigned)a_k[j] * 2u;
#pragma unroll
  for (int j = 0; j < kLoadsB; ++j) b_off[j] = (unsigned)b_row[j] * ldb + b_col[j];

  // Copies of k-step t into buffer buf: the A tile (kA), the B tile (kB) or both.  A
  // ragged last k-step is issued whole with the A part.
  constexpr int kA = 1, kB = 2;
  auto issue = [&](int t, int buf, int parts) __attribute__((always_inline)) {
    const int k0 = kbeg + t * kBK;
    char* sa = smem + buf * kStage;
    char* sb = sa + kATile;
    if (k0 + kBK <= K) {
      const char* ga = (const char*)p.a + (size_t)k0 * 2;
      const char* gb = (const char*)p.b + (size_t)k0 * ldb;
      if (parts & kA) {
#pragma unroll
        for (int j = 0; j < kLoadsA; ++j) copy_to_lds(ga, a_off[j], lds_addr(sa + (j * kWaves + wave) * 1024));
      }
      if (parts & kB) {
#pragma unroll
        for (int j = 0; j < kLoadsB; ++j) copy_to_lds(gb, b_off[j], lds_addr(sb + (j * kWaves + wave) * 1024));
      }
      return;
    }
    if (!(parts & kA)) return;
    // ragged last k-step: clamped offsets from the row bases
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
      // chunks past K read the last chunk of the row; zeroed after they land
      const unsigned off = a_row[j] + (unsigned)min(k0 + a_k[j], K - 8) * 2u;
      copy_to_lds(p.a, off, lds_addr(sa + (j * kWaves + wave) * 1024));
    }
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
      const unsigned off = (unsigned)min(k0 + b_row[j], K - 1) * ldb + b_col[j];
      copy_to_lds(p.b, off, lds_addr(sb + (j * kWaves + wave) * 1024));
    }
  };

  f32x16_t acc[kMB][kNB];
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < kNB; ++j) acc[i][j] = f32x16_t{};

  // LDS byte offsets of this lane's operands at k16 step 0 (step kc adds 2kc chunks of
  // A, 16 rows of B).
  unsigned a_op[kMB], b_op[kNB][2];
#pragma unroll
  for (int i = 0; i < kMB; ++i) a_op[i] = lds_off<8>(wave_m * (kMB * 32) + i * 32 + (lane & 31), G);
#pragma unroll
  for (int j = 0; j < kNB; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) b_op[j][h] = v_operand_off<kRB>(lane, wave_n * kNB + j, h);

  // k16 substeps [kc_lo, kc_hi) of a k-step
  auto compute = [&](const char* sa, const char* sb, int kc_lo, int kc_hi) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = kc_lo; kc < kc_hi; ++kc) {
      v8_t af[kMB], bf[kNB];
#pragma unroll
      for (int i = 0; i < kMB; ++i) {
        // chunk 2kc + G of the row: the R = 8 swizzle keeps chunk bits above bit 0 in
        // the slot's low bits, so stepping kc moves the slot by XOR, not by addition
        af[i] = *(const v8_t*)(sa + (a_op[i] ^ (unsigned)(kc << 5)));
      }
#pragma unroll
      for (int j = 0; j < kNB; ++j) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(sb + b_op[j][0] + kc * 16 * (kBN * 2)));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(sb + b_op[j][1] + kc * 16 * (kBN * 2)));
        bf[j] = __builtin_bit_cast(v8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = Mfma<T>::mma(bf[j], af[i], acc[i][j]);
    }
  };

  // step t of the workgroup's loop; a k-group with fewer k-steps than the loop (the
  // second group when their count is odd) only takes part in the barriers
  auto step = [&](int t, auto buf_tag) __attribute__((always_inline)) {
    const bool active = t < nk;
#if MHA_SERIALIZE
    // race-check form: one buffer, copied, waited for and fenced before it is read
    constexpr int buf = 0;
    (void)buf_tag;
    tile_barrier();
    if (active) issue(t, 0, kA | kB);
#else
    constexpr int buf = decltype(buf_tag)::value;
#endif
    char* sa = smem + buf * kStage;
    wait_vmcnt<0>();
    const int k0 = kbeg + t * kBK;
    if (active && k0 + kBK > K) {
      // ragged last k-step: zero the A chunks past K that this thread copied
#pragma unroll
      for (int j = 0; j < kLoadsA; ++j)
        if (k0 + a_k[j] >= K) *(uint4*)(sa + (j * kWaves + wave) * 1024 + lane * 16) = uint4{0, 0, 0, 0};
    }
    tile_barrier();
    if (!active) return;
#if MHA_SERIALIZE
    compute(sa, sa + kATile, 0, kBK / 16);
#else
    // the next step's copies go out between the first MFMAs of this one (measured: up
    // to a quarter faster than issuing them all before the first MFMA)
    compute(sa, sa + kATile, 0, 1);
    if (t + 1 < nk) issue(t + 1, buf ^ 1, kA);
    compute(sa, sa + kATile, 1, 2);
    if (t + 1 < nk) issue(t + 1, buf ^ 1, kB);
    compute(sa, sa + kATile, 2, kBK / 16);
#endif
  };

#if !MHA_SERIALIZE
  if (nk > 0) issue(0, 0, kA | kB);
#endif
  for (int t = 0; t < nsteps; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nsteps) step(t + 1, std::integral_constant<int, 1>{});
  }

  if constexpr (kKG > 1) {
    // group 1 hands its sums to group 0 through its own (now idle) stages: wavefront w
    // of group 1 writes its accumulators lane-contiguously, wavefront w of group 0 (same
    // block of C) adds them.  The barriers order the group's last operand reads before
    // the writes, and the writes before the reads.
    constexpr int kRegs = kMB * kNB * 16;
    float* xfer = (float*)(lds + 2 * kStage) + (size_t)wave * kRegs * 64;
    tile_barrier();
    if (kgrp == 1) {
#pragma unroll
      for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
            *(f32x4_t*)(xfer + (((i * kNB + j) * 4 + q) * 64 + lane) * 4) = v;
          }
    }
    tile_barrier();
    if (kgrp == 1) return;
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t v = *(const f32x4_t*)(xfer + (((i * kNB + j) * 4 + q) * 64 + lane) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] += v[e];
        }
  }

  // --- epilogue: register r of block (i, j) is row (lane & 31) of the block and
  // column 32j + 16(r >> 3) + 8G + (r & 7).
  if constexpr (SPLITK) {
    // float32 partial block of this split
    const int split = kbeg / p.kchunk;
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
      const int m = m0 + wave_m * (kMB * 32) + i * 32 + (lane & 31);
      if (m >= M) continue;
      float* prow = p.part + ((size_t)split * M + m) * N;
#pragma unroll
      for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int n = n0 + wave_n * (kNB * 32) + j * 32 + 16 * hh + 8 * G;
          if (n >= N) continue;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            f32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][8 * hh + 4 * q + e];
            *(f32x4_t*)(prow + n + 4 * q) = v;
          }
        }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kMB; ++i) {
    const int m = m0 + wave_m * (kMB * 32) + i * 32 + (lane & 31);
    if (m >= M) continue;
    T* crow = (T*)p.c + (size_t)m * N;
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int n = n0 + wave_n * (kNB * 32) + j * 32 + 16 * hh + 8 * G;
        if (n >= N) continue;
        typename Mfma<T>::v8 ov;
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = (T)acc[i][j][8 * hh + e];
        *(typename Mfma<T>::v8*)(crow + n) = ov;
      }
  }
}

// C = sum over splits of the float32 partials, rounded once to T.  Thread i owns the 8
// consecutive elements 8i .. 8i+7 of C (N is a multiple of 8, so they share a row).
constexpr int kReduceThreads = 256;
template <typename T>
__global__ __launch_bounds__(kReduceThreads) void gemm_splitk_reduce(GemmParams p) {
  const size_t total = (size_t)p.M * p.N;
  const size_t i = ((size_t)blockIdx.x * kReduceThreads + threadIdx.x) * 8;
  if (i >= total) return;
  f32x4_t lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.splits; ++s) {
    const float* src = p.part + (size_t)s * total + i;
    lo += *(const f32x4_t*)src;
    hi += *(const f32x4_t*)(src + 4);
  }
  typename Mfma<T>::v8 ov;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ov[e] = (T)lo[e];
    ov[4 + e] = (T)hi[e];
  }
  *(typename Mfma<T>::v8*)((T*)p.c + i) = ov;
}

template <typename C>
void launch_tiled(GemmParams p, int dtype, hipStream_t stream) {
  p.tiles_m = (p.M + C::BM - 1) / C::BM;
  p.tiles_n = (p.N + C::BN - 1) / C::BN;
  p.total = p.tiles_m * p.tiles_n;
  if (dtype == 2)
    hipLaunchKernelGGL((gemm_kernel<_Float16, C>), dim3(p.total), dim3(C::Threads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<__bf16, C>), dim3(p.total), dim3(C::Threads), 0, stream, p);
}

// 0: the 256 x 256 tiling, 1: 128 x 128, 2: 128 x 64, 3: 128 x 128 with two k-groups.
int gemm_tiling(int M, int N, int K) {
  const long large = (long)((M + Large::BM - 1) / Large::BM) * ((N + Large::BN - 1) / Large::BN);
  if (large >= kLargeMinTiles) return 0;
  const long small = (long)((M + Small::BM - 1) / Small::BM) * ((N + Small::BN - 1) / Small::BN);
  if (small >= kSmallMinTiles) return 1;
  return K >= kDuoMinK ? 3 : 2;
}

}  // namespace

hipError_t launch_gemm(const void* a, const void* b, void* c, int M, int N, int K, int dtype,
                       hipStream_t stream) {
  GemmParams p;
  p.a = a;
  p.b = b;
  p.c = c;
  p.M = M;
  p.N = N;
  p.K = K;
  const int tiling = gemm_tiling(M, N, K);
  if (tiling == 0)
    launch_tiled<Large>(p, dtype, stream);
  else if (tiling == 1)
    launch_tiled<Small>(p, dtype, stream);
  else if (tiling == 2)
    launch_tiled<Tiny>(p, dtype, stream);
  else
    launch_tiled<Duo>(p, dtype, stream);
  return hipGetLastError();
}

hipError_t launch_gemm_splitk(const void* a, const void* b, void* c, int M, int N, int K, int dtype, int splits,
                              int kchunk, float* part, hipStream_t stream) {
  GemmParams p;
  p.a = a;
  p.b = b;
  p.c = c;
  p.M = M;
  p.N = N;
  p.K = K;
  p.kchunk = kchunk;
  p.splits = splits;
  p.part = part;
  p.tiles_m = (M + Small::BM - 1) / Small::BM;
  p.tiles_n = (N + Small::BN - 1) / Small::BN;
  p.total = p.tiles_m * p.tiles_n;
  const dim3 grid(p.total * splits);
  const dim3 rgrid((unsigned)(((size_t)M * N / 8 + kReduceThreads - 1) / kReduceThreads));
  if (dtype == 2) {
    hipLaunchKernelGGL((gemm_kernel<_Float16, Small, true>), grid, dim3(Small::Threads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_splitk_reduce<_Float16>), rgrid, dim3(kReduceThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((gemm_kernel<__bf16, Small, true>), grid, dim3(Small::Threads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_splitk_reduce<__bf16>), rgrid, dim3(kReduceThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mha_impl
