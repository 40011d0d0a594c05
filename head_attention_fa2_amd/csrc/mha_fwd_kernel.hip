// Fused multi-head attention forward for gfx950 (AMD Instinct MI355X, CDNA4).
//
// Computes Algorithm 1 ("FlashAttention-2 forward") of "ML-Triton, A Multi-Level
// Compilation and Language Extension to Triton GPU Programming", section 2.5: for each
// (batch, head) the query rows are split into blocks; a block loads its Q rows once,
// then streams K/V tiles, forms S = Q.K_j^T, updates the running row max m and row sum
// l with the online softmax (the running-sum update of the "Long Softmax" puzzle in
// "Triton学习", lorn3.bearblog.dev), accumulates O += P.V_j, and stores O / l and the
// logsumexp m + ln l once at the end.  The work partition is the one section 2.5 takes
// from FlashAttention-2: output rows are distributed over the wavefronts and every
// wavefront reads all of K/V, so wavefronts never exchange partial results.
//
// Mapping onto CDNA4:
//  * A workgroup of 4 wavefronts owns 128 query rows, 32 per wavefront; three
//    workgroups (12 wavefronts, 3 per SIMD) share a CU at d = 128 on 16-bit inputs, up
//    to four at d = 64.  A wavefront raises its issue priority (s_setprio) while it
//    feeds the matrix cores with independent MFMAs and drops it for the softmax, so the
//    other wavefronts of the SIMD fill the MFMA shadow with VALU work.
//  * Both contractions are v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2_f32).
//    The scores are formed transposed, S^T = K.Q^T, so that the 32 lanes of a column
//    each own ONE query row: row max / row sum are in-lane reductions plus one
//    exchange between lane n and lane n+32 (v_permlane32_swap).  Output likewise is
//    O^T = V^T.P^T, so the per-row rescale and 1/l are in-lane multiplies.
//  * K rows enter the first product in an order that swaps bits 2 and 3 of the row
//    index inside each 32-row slab; the fp32 accumulator of S^T is then, register for
//    register, the bf16 B operand P^T of the second product (8 consecutive keys per
//    lane half), so P needs no cross-lane shuffle.
//  * K/V tiles (32 keys at d = 128 on 16-bit inputs, else 64) are copied HBM -> LDS
//    with global_load_lds_dwordx4 (no VGPR
//    staging), double buffered with one barrier per tile: after the barrier of step j
//    every wavefront has finished step j-1, so tile j+1 is copied into that buffer and
//    stays in flight while tile j is consumed.
//    LDS rows are XOR-swizzled in 16-byte chunks so that the MFMA operand reads of
//    K (ds_read_b128) and of V^T (ds_read_b64_tr_b16, the gfx950 transposing LDS read)
//    are free of bank conflicts.
//  * exp is evaluated as exp2 with the scale folded into one FMA (log2(e) prescale, as
//    the "Long Softmax" puzzle recommends).  The exponent offset is lazy: it is set to
//    the row max on a wavefront's first tile and afterwards only moved when a tile's
//    exponentials grow large (a lane's sum of them above 2^24, or 2^15 for fp16), so
//    most tiles take no row max at all and O and l are rarely rescaled; the final O / l
//    and m + ln l are exact for whichever offset was used.
//  * Causal: key tiles entirely above a wavefront's rows are skipped, only tiles that
//    cross the diagonal (or the ragged end of the sequence) evaluate the mask, and
//    heavy (late) query blocks are dispatched first.  Workgroup ids are
//    remapped so that all query blocks of a head run on the same XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "gfx950_lds.h"
#include "mha_launch.h"
#include "mha_layout.h"

// copy_to_lds sets m0 itself right before each copy; nothing else in these kernels
// reads m0, so declaring it clobbered is sound.
#pragma clang diagnostic ignored "-Winline-asm"

// MHA_SERIALIZE=1 builds the race-check form of the tile loop: one LDS buffer, and every
// tile is copied, waited for and fenced by a barrier before any wavefront reads it, with a
// second barrier before the next copy overwrites it.  No copy is ever in flight while
// operands are read, and the arithmetic (and its order) is unchanged, so its results must
// equal the pipelined kernel's bit for bit.
#ifndef MHA_SERIALIZE
#define MHA_SERIALIZE 0
#endif

namespace mha_impl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// 16-bit element types: the 8-element operand vector and the 32x32x16 MFMA that
// consumes it (fp32 accumulate).  fp32 inputs use the fp32 MFMA paths instead.
template <typename T>
struct Half16 {
  typedef bf16x8_t v8;   // unused for fp32
};
template <>
struct Half16<__bf16> {
  typedef bf16x8_t v8;
  static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Half16<_Float16> {
  typedef f16x8_t v8;
  static __device__ __forceinline__ f32x16_t mma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kQW = 32;                  // query rows per wavefront
// Keys per K/V tile: 32 for the fused kernel on 16-bit inputs with d = 128 (a 32 KiB
// double-buffered tile set and 160-165 VGPRs let three workgroups share a CU; measured +1-4 %
// on d = 128 against 64-key tiles at two workgroups per CU, but -4 % at d = 64), 64
// otherwise (split-KV and paged kernels included).
template <typename T, int D, bool SPLIT>
constexpr int tile_keys() { return sizeof(T) == 2 && D == 128 && !SPLIT ? 32 : 64; }
constexpr int kWaves = 4;                // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kQW * kWaves;        // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy offset: a tile's exponentials are taken against the current offset, and the
// offset is only moved (the tile's scores formed again and its row max taken) when some
// lane's sum of them exceeds this bound, so every exponential used is at most the bound:
// 2^24 (the accumulated O then stays below Nk * 2^24 * max|v|, inside the float32 range
// while Nk * max|v| < 2^100), and 2^15 when P is rounded to float16, whose largest value
// is 65504.
template <typename T>
constexpr float sum_limit() { return std::is_same<T, _Float16>::value ? 32768.0f : 16777216.0f; }
constexpr int kOrderHeads = 4;           // causal: heads per ordering group on an XCD

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;          // query rows per head (= keys per head, except for the split-KV kernel)
  int nqb;        // query blocks per head
  int total;      // workgroups
  float qmul;     // sign(scale): Q is multiplied by it on load (1, -1 or 0)
  float scale2;   // |scale| * log2(e), or log2(e) when scale == 0
  // split-KV only: keys per head, keys per split (a multiple of the tile), number of
  // splits, B*H, and the float32 partial results [split][B*H][N][d] and [split][B*H][N]
  int Nk;
  int chunk;
  int splits;
  int BH;
  float* part_o;
  float* part_lse;
  // paged K/V only: heads, block table [B][max_blocks] and key counts [B] (int32), pool
  // size in blocks, log2 of the block size (keys per block)
  int H = 0;
  const int* block_table = nullptr;
  const int* seq_lens = nullptr;  // also tells the merge that key counts vary per sequence
  int max_blocks = 0;
  int num_blocks = 0;
  int bs_log2 = 0;
};

// ---------------------------------------------------------------------------- LDS layout
// Chunk swizzle, its inverse and the slab row permutation live in mha_layout.h.
using mha_layout::lds_inv;
using mha_layout::lds_off;
using mha_layout::sigma;

// Exchange with lane (l ^ 32): returns (own, partner) folded by max / sum.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  // a and b hold the same value on entry; afterwards lanes 0-31 have (own, partner's)
  // and lanes 32-63 have (partner's, own) in (a, b).
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_halves(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

using gfx950::copy_to_lds;
using gfx950::copy_to_lds_addr;
using gfx950::lds_addr;
using gfx950::tile_barrier;
using gfx950::uniform_ptr;
using gfx950::wait_vmcnt;

// ---------------------------------------------------------------------------- kernel
// Occupancy the register allocation must allow (wavefronts per SIMD = workgroups per
// CU): three for the 32-key tiles (32 KiB of LDS, at most 168 VGPRs), two when the
// double-buffered 64-key tiles fit twice in the 160 KiB of LDS, else one (fp32 with
// d = 128 needs 128 KiB).  Kernels that need fewer registers may run more (d = 64 on
// 16-bit inputs: four).
template <typename T, int D, bool SPLIT, bool KSPLIT = false>
constexpr int min_waves_per_eu() {
  constexpr int keys = tile_keys<T, D, SPLIT>();
  if constexpr (KSPLIT) return D == 64 ? 4 : 2;   // 8-wavefront workgroups: up to two per CU at d = 64, one at d = 128
  return keys == 32 ? 3 : 2 * 2 * keys * D * (int)sizeof(T) <= 80 * 1024 ? 2 : 1;
}

// KSPLIT (fused forward on 16-bit inputs, for grids too small to fill the CUs): a workgroup
// of 8 wavefronts in two groups of 4; both groups own the same 128 query rows, group 0
// streams the first half of the key tiles and group 1 the second, each through its own
// double-buffered LDS tiles, and group 1 hands its (O, l, offset) to group 0 through LDS
// at the end, where they are merged exactly as two key ranges of the online softmax are:
// offset m = max(m0, m1), O = O0 2^(c(m0-m)) + O1 2^(c(m1-m)), l likewise.
template <typename T, int D, bool SPLIT, bool KSPLIT>
constexpr int lds_bytes() {
  constexpr int tile = tile_keys<T, D, SPLIT>() * D * (int)sizeof(T);
  if constexpr (!KSPLIT) return 2 * 2 * tile;
  constexpr int stages = 2 * 2 * 2 * tile;                       // [group][buf][K,V]
  constexpr int merge = kWaves * ((D / 32) * 16 + 2) * 64 * 4;   // group 1's O, offset, l
  return stages > merge ? stages : merge;
}

// SPLIT: the split-KV form (no mask): workgroup (split, head, query block) covers the
// keys [split * chunk, min(Nk, (split + 1) * chunk)) and writes its O (normalised by its
// own l) and logsumexp to the float32 partial buffers; mha_merge_kernel combines them.
// PAGED (with SPLIT): K and V are gathered from block pools [num_blocks][H][bs][d]
// through the block table; head b*H + h uses keys [0, seq_lens[b]).
template <typename T, int D, bool CAUSAL, bool SPLIT = false, bool PAGED = false, bool KSPLIT = false>
__global__ __launch_bounds__(KSPLIT ? 2 * kThreads : kThreads)
__attribute__((amdgpu_waves_per_eu(min_waves_per_eu<T, D, SPLIT, KSPLIT>())))
void mha_fwd_kernel(Params p) {
  static_assert(!(SPLIT && CAUSAL), "the split-KV form has no mask");
  static_assert(!PAGED || SPLIT, "paged K/V uses the split-KV form");
  static_assert(!KSPLIT || (!SPLIT && sizeof(T) == 2), "key halves per workgroup: fused forward, 16-bit");
  constexpr int kBN = tile_keys<T, D, SPLIT>();  // keys per K/V tile
  constexpr int kSlabs = kBN / 32;               // 32-key MFMA slabs per tile
  constexpr bool k16 = sizeof(T) == 2;         // bf16 or fp16 inputs
  typedef typename Half16<T>::v8 h8_t;
  constexpr int RB = D * (int)sizeof(T);        // bytes per K/V row
  constexpr int R = RB / 16;                     // 16-byte chunks per row
  constexpr int kTileBytes = kBN * RB;
  constexpr int kLoads = kBN * R / kThreads;     // 16-byte loads per thread per tile
  static_assert(kLoads * kThreads == kBN * R, "tile must split evenly");
  static_assert(lds_bytes<T, D, SPLIT, KSPLIT>() >= (KSPLIT ? 2 : 1) * 2 * 2 * kTileBytes, "LDS stages");
  constexpr int kDT = D / 32;                    // 32-wide output column blocks

  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<T, D, SPLIT, KSPLIT>()];  // [group][buf][K,V]

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kgrp = KSPLIT ? wave_all >> 2 : 0;  // key half of this wavefront (KSPLIT)
  const int wave = wave_all - kgrp * kWaves;    // wavefront within its group: its query rows
  char* const smem = lds + kgrp * 2 * 2 * kTileBytes;
  const int n = lane & 31;      // query column (and K row slot) within the wavefront
  const int G = lane >> 5;      // lane half

  // --- workgroup -> (head, query block).  Consecutive workgroup ids go to different
  // XCDs, so renumber: the k-th workgroup dispatched to XCD x gets task x*T/8 + k, which
  // keeps every head's query blocks on one XCD (they share its L2).
  int id = blockIdx.x;
  if ((p.total & 7) == 0) id = (id & 7) * (p.total >> 3) + (id >> 3);
  int split = 0;
  if constexpr (SPLIT) {
    split = id / (p.nqb * p.BH);
    id -= split * p.nqb * p.BH;
  }
  int bh = id / p.nqb;
  int qb = id - bh * p.nqb;          // dispatch rank within the head; causal: 0 = heaviest
  if constexpr (CAUSAL) {
    // Causal blocks differ in work (block qb sees (qb + 1) * kBM keys).  Taken head after
    // head, the heaviest blocks of an XCD's last heads would start near the end and leave
    // CUs idle in a long tail.  So when B*H is a multiple of 8 (each XCD owns whole heads
    // [x*hx, (x+1)*hx)), an XCD runs its heads in groups of kOrderHeads, and inside a
    // group the heaviest block of every head first, then the next heaviest, and so on.
    // The blocks of one group's heads still run close together in time, so their K/V
    // tiles are mostly read once into the XCD's L2.
    const int BH = p.total / p.nqb;
    if ((BH & 7) == 0) {
      const int hx = BH >> 3, x = blockIdx.x & 7, k = blockIdx.x >> 3;
      const int grp = k / (kOrderHeads * p.nqb);
      const int r = k - grp * kOrderHeads * p.nqb;
      const int gs = min(kOrderHeads, hx - grp * kOrderHeads);   // heads in this group
      const int rank = r / gs;
      bh = x * hx + grp * kOrderHeads + (r - rank * gs);
      qb = rank;
    }
    qb = p.nqb - 1 - qb;
  }
  const int N = p.N;                            // query rows
  int seq_b = 0, head_h = 0;                    // paged: sequence and head of this workgroup
  int Nk = SPLIT ? p.Nk : N;                    // keys
  if constexpr (PAGED) {
    seq_b = bh / p.H;
    head_h = bh - seq_b * p.H;
    Nk = min(max(p.seq_lens[seq_b], 0), p.max_blocks << p.bs_log2);
  }
  int kbeg = SPLIT ? split * p.chunk : 0;       // this workgroup's keys: [kbeg, kend)
  const int kend = SPLIT ? min(Nk, kbeg + p.chunk) : N;
  const int q0 = qb * kBM;
  const int qw = q0 + wave * kQW;               // first query row of this wavefront
  const int qrow = qw + n;                      // the query row this lane owns
  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t khead = SPLIT ? (size_t)bh * (size_t)Nk * D : head;
  const T* __restrict__ Q = (const T*)p.q + head;
  const char* Kbase = (const char*)((const T*)p.k + khead);
  const char* Vbase = (const char*)((const T*)p.v + khead);

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : kend;
  int ntiles = PAGED ? max(0, (kv_end - kbeg + kBN - 1) / kBN) : (kv_end - kbeg + kBN - 1) / kBN;
  int nsteps = ntiles;                          // steps of the loop (every wavefront's barriers)
  if constexpr (KSPLIT) {
    // group 0: tiles [0, h), group 1: tiles [h, ntiles)
    const int h = (ntiles + 1) / 2;
    nsteps = h;
    if (kgrp == 1) {
      kbeg = h * kBN;
      ntiles -= h;
    } else {
      ntiles = h;
    }
  }
  // paged: a key range that starts past this sequence's end has nothing to do; the merge
  // reads only the ranges below the sequence's key count.  With a single range (no
  // merge) an empty sequence's rows are written here: O = 0 and lse = log 0 = -inf.
  if (PAGED && ntiles == 0) {
    if (p.splits == 1 && qrow < N) {
      T* orow = (T*)p.o + head + (size_t)qrow * D;
#pragma unroll
      for (int c = G * (D / 2); c < (G + 1) * (D / 2); c += 16 / (int)sizeof(T)) *(f32x4_t*)(orow + c) = f32x4_t{};
      if (G == 0) p.lse[(size_t)bh * N + qrow] = -__builtin_inff();
    }
    return;
  }

  // --- tile loader: thread (wave, lane) copies kLoads 16-byte chunks of K and of V.
  // Load j of a thread fills LDS bytes [(j*kWaves + wave)*1024, +1024); the swizzle is
  // periodic in the row index, so the global row of load j is row0 + j*kRowStep and
  // its chunk is the same for every j.
  constexpr int kRowStep = 1024 * kWaves / RB;
  int ld_row[kLoads], ld_chunk[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    if (mha_layout::loader_periodic<R>() && j > 0) {
      ld_row[j] = ld_row[0] + j * kRowStep;
      ld_chunk[j] = ld_chunk[0];
    } else {
      lds_inv<R>((j * kWaves + wave) * 64 + lane, ld_row[j], ld_chunk[j]);
    }
  }
  const int ld_row0 = ld_row[0];
  const unsigned ld_off0 = (unsigned)(ld_row0 * RB + ld_chunk[0] * 16);

  // --- paged K/V: key j of this sequence is row j % bs of block table[j / bs], and a
  // block holds, per head, bs contiguous rows.  The table entries of a tile are read one
  // step before its copies are issued, into ent[], with plain loads that the vmcnt(0)
  // wait opening every step covers.  With bs >= kBN a tile (kBN-aligned) lies inside one
  // block: one entry, a uniform base and the usual offsets.  Smaller blocks take one
  // entry and a 64-bit address per copied row.  Entries are clamped into the pool, so a
  // bad table gives wrong values, never an access outside the pools.
  int ent[kLoads];
  const int* btab = nullptr;
  int bsl = 0;
  if constexpr (PAGED) btab = p.block_table + (size_t)seq_b * p.max_blocks;
  if constexpr (PAGED) bsl = p.bs_log2;
  const bool big_blocks = bsl >= 6;
  auto fetch_entries = [&](int t) __attribute__((always_inline)) {
    const int k0 = kbeg + t * kBN;
    if (big_blocks) {
      ent[0] = btab[min(k0 + ld_row0, kend - 1) >> bsl];
    } else {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) ent[j] = btab[min(k0 + ld_row[j], kend - 1) >> bsl];
    }
  };
  // byte offset in a pool of row `key` (of this sequence and head) stored in block blk
  auto pool_offset = [&](int blk, int key) __attribute__((always_inline)) {
    blk = min(max(blk, 0), p.num_blocks - 1);
    return ((((size_t)blk * p.H + head_h) << bsl) + (size_t)(key & ((1 << bsl) - 1))) * RB;
  };

  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const int k0 = kbeg + t * kBN;
    const char* kg = Kbase + (size_t)k0 * RB;
    const char* vg = Vbase + (size_t)k0 * RB;
    char* lk = smem + buf * 2 * kTileBytes;
    char* lv = lk + kTileBytes;
    if constexpr (PAGED) {
      if (!big_blocks) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          const size_t off = pool_offset(ent[j], min(k0 + ld_row[j], kend - 1)) + ld_chunk[j] * 16;
          const int dst = (j * kWaves + wave) * 1024;
          copy_to_lds_addr((const char*)p.k + off, lds_addr(lk + dst));
          copy_to_lds_addr((const char*)p.v + off, lds_addr(lv + dst));
        }
        return;
      }
      const size_t base = pool_offset(__builtin_amdgcn_readfirstlane(ent[0]), k0);
      kg = uniform_ptr((const char*)p.k + base);
      vg = uniform_ptr((const char*)p.v + base);
    }
    if (k0 + kBN <= kend) {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const unsigned off = mha_layout::loader_periodic<R>()
                                 ? ld_off0 + (unsigned)(j * kRowStep * RB)
                                 : (unsigned)(ld_row[j] * RB + ld_chunk[j] * 16);
        const int dst = (j * kWaves + wave) * 1024;
        copy_to_lds(kg, off, lds_addr(lk + dst));
        copy_to_lds(vg, off, lds_addr(lv + dst));
      }
    } else {
      // ragged last tile: rows past the end re-read the last key (finite, masked later)
      const int last = kend - 1 - k0;   // (uniform: no per-tile update of per-lane rows)
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int row = min(ld_row[j], last);
        const unsigned off = (unsigned)(row * RB + ld_chunk[j] * 16);
        const int dst = (j * kWaves + wave) * 1024;
        copy_to_lds(kg, off, lds_addr(lk + dst));
        copy_to_lds(vg, off, lds_addr(lv + dst));
      }
    }
  };

  // --- Q operand, kept in registers for the whole loop ("Load Q" once).
  // bf16: lane (n, G) holds Q[qrow][16kc + 8G .. +7] for kc = 0..D/16-1.
  // fp32: lane (n, G) holds Q[qrow][8j + 4G .. +3] for j = 0..D/8-1.
  constexpr int kQF = k16 ? D / 16 : D / 8;
  typedef typename std::conditional<k16, h8_t, f32x4_t>::type qfrag_t;
  qfrag_t qf[kQF];
  {
    const bool valid = qrow < N;
    const T* qr = Q + (size_t)(valid ? qrow : 0) * D;
#pragma unroll
    for (int j = 0; j < kQF; ++j) {
      const int col = k16 ? 16 * j + 8 * G : 8 * j + 4 * G;
      qf[j] = *(const qfrag_t*)(qr + col);
      if (!valid) qf[j] = qfrag_t{};
      // scaled logit = scale * q.k = |scale| * (sign(scale) q).k; multiplying by 1, -1
      // or 0 is exact, so the row max below is always taken on the logit's own order.
#pragma unroll
      for (int e = 0; e < (int)(sizeof(qfrag_t) / sizeof(T)); ++e) qf[j][e] = (T)((float)qf[j][e] * p.qmul);
    }
  }

  // --- per-lane LDS offsets of the MFMA operands (constant over tiles).
  // K (A operand of S^T): lane (n, G) reads key row sigma(n) (+32 per slab), chunk
  // 2kc + G.  Same chunk rule for both element types (8 bf16 or 4 fp32 per chunk).
  constexpr int kKF = kQF;
  int offK[kKF];
#pragma unroll
  for (int j = 0; j < kKF; ++j) offK[j] = mha_layout::k_operand_off<R>(lane, j);
  // V^T (A operand of O^T, bf16): ds_read_b64_tr_b16 gathers, in each 16-lane group, a
  // 4-key x 16-column block; source lane s supplies key (s >> 2) and the 4-column group
  // chosen so that output lane m ends up with column sigma(m).
  int offV[k16 ? kDT : 1][2];
  if constexpr (k16) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) offV[dt][h] = mha_layout::v_operand_off<R>(lane, dt, h);
  }

  // --- running state: this lane's query row.
  f32x16_t acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = f32x16_t{};
  float m_run = -__builtin_inff();   // exponent offset in raw score units
  float mc = 0.f;                    // m_run * c2 once set
  float l_run = 0.f;                 // this lane's share of the row sum
  bool fresh = true;                 // no tile consumed yet: the offset is unset
  const float c2 = p.scale2;

  // S^T = K_j . Q^T for the tile at lk (keys k0..), masked when `masked`.
  auto scores = [&](f32x16_t (&s)[kSlabs], const char* lk, int k0, bool masked) __attribute__((always_inline)) {
    // One or two 32-key slabs, accumulated in alternation so consecutive MFMAs are
    // independent; K operands are read two steps ahead.  With two slabs the wavefront
    // raises its issue priority for these MFMAs, as for P.V below; a single slab is one
    // dependent MFMA chain, and raising the priority there only holds back the other
    // wavefronts' softmax while the chain waits on itself (measured +1-2 % at d = 128
    // without it).
#pragma unroll
    for (int ks = 0; ks < kSlabs; ++ks) s[ks] = f32x16_t{};
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kSlabs == 2) __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (k16) {
      constexpr int KC = D / 16;
      h8_t kf[KC][kSlabs];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int ks = 0; ks < kSlabs; ++ks) kf[kc][ks] = *(const h8_t*)(lk + offK[kc] + ks * 32 * RB);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int ks = 0; ks < kSlabs; ++ks)
          s[ks] = Half16<T>::mma(kf[kc][ks], qf[kc], s[ks]);
      // schedule: 2 steps of reads, then (one step of MFMAs, one of reads) ..., then the
      // last MFMAs (a step: one per slab)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kSlabs, 0);
#pragma unroll
      for (int i = 0; i < KC - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, kSlabs, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kSlabs, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kSlabs, 0);
    } else {
#pragma unroll
      for (int j = 0; j < D / 8; ++j)
#pragma unroll
        for (int ks = 0; ks < kSlabs; ++ks) {
          const f32x4_t kf = *(const f32x4_t*)(lk + offK[j] + ks * 32 * RB);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            s[ks] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[t], qf[j][t], s[ks], 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kSlabs == 2) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    // Mask: accumulator register r of slab ks on lane half G is key
    // k0 + 32ks + 16(r>>3) + 8G + (r&7).
    if (masked) {
      const int lim = CAUSAL ? min(qrow, N - 1) : kend - 1;
      const int rel = lim - k0 - 8 * G;   // key > lim  <=>  32ks + 16(r>>3) + (r&7) > rel
#pragma unroll
      for (int ks = 0; ks < kSlabs; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * ks + 16 * (r >> 3) + (r & 7) > rel) s[ks][r] = -__builtin_inff();
    }
  };

  // Online softmax (running max / sum of the "Long Softmax" puzzle), offset update: the
  // tile's row max (three-way maxima in a tree, then the exchange between the two lane
  // halves) becomes the offset if it is larger, and O and l are rescaled to it.  Every
  // row has a visible key in a wavefront's first tile, so the offset is finite after it.
  auto rebase = [&](const f32x16_t (&s)[kSlabs]) __attribute__((always_inline)) {
    float part[kSlabs][6];
#pragma unroll
    for (int ks = 0; ks < kSlabs; ++ks) {
#pragma unroll
      for (int g = 0; g < 5; ++g) part[ks][g] = fmaxf(fmaxf(s[ks][3 * g], s[ks][3 * g + 1]), s[ks][3 * g + 2]);
      part[ks][5] = s[ks][15];
    }
    float mx = fmaxf(fmaxf(part[0][0], part[0][1]), part[0][5]);
    float my = fmaxf(fmaxf(part[0][2], part[0][3]), part[0][4]);
#pragma unroll
    for (int ks = 1; ks < kSlabs; ++ks) {
      mx = fmaxf(fmaxf(mx, part[ks][0]), fmaxf(part[ks][1], part[ks][5]));
      my = fmaxf(fmaxf(my, part[ks][2]), fmaxf(part[ks][3], part[ks][4]));
    }
    mx = max_halves(fmaxf(mx, my));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2((m_run - m_new) * c2);    // 0 when m_run = -inf
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) acc[dt] *= alpha;
    m_run = m_new;
    mc = m_new * c2;
  };

  // P = exp2(c2 * s - offset) in place; returns this lane's sum of them.
  auto exponentials = [&](f32x16_t (&s)[kSlabs]) __attribute__((always_inline)) {
    float la, lb;   // two partial sums: half the dependent-add chain
#pragma unroll
    for (int ks = 0; ks < kSlabs; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(s[ks][r], c2, -mc));
        s[ks][r] = e;
        if (ks == 0 && r < 2) (r ? lb : la) = e;
        else (r & 1 ? lb : la) += e;
      }
    return la + lb;
  };

  auto compute_tile = [&](const char* lk, const char* lv, int k0, bool masked) __attribute__((always_inline)) {
    f32x16_t s[kSlabs];
    scores(s, lk, k0, masked);
    if (fresh) {
      rebase(s);
      fresh = false;
    }
    // The offset stays put while the exponentials stay small: no row max on such tiles.
    // A lane sum above sum_limit (a key far above the offset; inf on overflow) sends the
    // whole wavefront back to form the tile's scores again from the LDS tile, move the
    // offset to the row max and exponentiate again (every value then at most 1).
    float ls = exponentials(s);
    if (__builtin_amdgcn_ballot_w64(ls > sum_limit<T>())) {
      scores(s, lk, k0, masked);
      rebase(s);
      ls = exponentials(s);
    }
    l_run += ls;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V_j^T . P^T
    if constexpr (k16) {
      h8_t pf[2 * kSlabs];   // P^T operand for key chunks kc2 = 2ks + hh (16 keys each)
#pragma unroll
      for (int ks = 0; ks < kSlabs; ++ks)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[2 * ks + hh][e] = (T)s[ks][8 * hh + e];
      h8_t vf[2 * kSlabs][kDT];
#pragma unroll
      for (int kc2 = 0; kc2 < 2 * kSlabs; ++kc2)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(lv + offV[dt][0] + kc2 * 16 * RB));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(lv + offV[dt][1] + kc2 * 16 * RB));
          vf[kc2][dt] = __builtin_bit_cast(h8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
      for (int kc2 = 0; kc2 < 2 * kSlabs; ++kc2)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
          acc[dt] = Half16<T>::mma(vf[kc2][dt], pf[kc2], acc[dt]);
      // schedule: 8 reads (4 operands), then (1 MFMA, 2 reads) ..., then the last MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 2 * kSlabs * kDT - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    } else {
      // fp32: two keys per MFMA.  B operand = P value in register u of slab ks (key
      // 32ks + 16(u>>3) + 8G + (u&7)); A operand on lane (m, G) = V[that key][32dt + m].
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int ks = 0; ks < kSlabs; ++ks)
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int key = 32 * ks + 16 * (u >> 3) + 8 * G + (u & 7);
            const int col = dt * 32 + n;
            const float vv = *(const float*)(lv + lds_off<R>(key, col >> 2) + (col & 3) * 4);
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, s[ks][u], acc[dt], 0, 0, 0);
          }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  // --- main loop over K/V tiles, double buffered, one barrier per tile.  Unrolled by
  // two so that the LDS buffer of each step is a compile-time address.
  auto step = [&](int t, auto buf_tag) __attribute__((always_inline)) {
#if MHA_SERIALIZE
    constexpr int buf = 0;
    (void)buf_tag;
    tile_barrier();                                    // every wavefront is done with tile t-1
    if constexpr (PAGED) fetch_entries(t);
    if (!KSPLIT || t < ntiles) issue_tile(t, 0);
    wait_vmcnt<0>();
    tile_barrier();                                    // tile t has landed for every wavefront
#else
    constexpr int buf = decltype(buf_tag)::value;
    wait_vmcnt<0>();
    tile_barrier();
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
    if constexpr (PAGED) {
      if (t + 2 < ntiles) fetch_entries(t + 2);
    }
#endif
    const int k0 = kbeg + t * kBN;
    if (KSPLIT && t >= ntiles) return;                 // this key half has no tile t
    if (SPLIT && qw >= N) return;                      // no query row in this wavefront
    if (!CAUSAL || k0 <= qw + kQW - 1) {               // else: every key is after every row
      const bool need_mask = (k0 + kBN > kend) || (CAUSAL && k0 + kBN - 1 > qw);
      compute_tile(smem + buf * 2 * kTileBytes, smem + buf * 2 * kTileBytes + kTileBytes, k0, need_mask);
    }
  };
#if !MHA_SERIALIZE
  if constexpr (PAGED) fetch_entries(0);
  if (!KSPLIT || ntiles > 0) issue_tile(0, 0);
  if constexpr (PAGED) {
    if (ntiles > 1) fetch_entries(1);
  }
#endif
  for (int t = 0; t < nsteps; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nsteps) step(t + 1, std::integral_constant<int, 1>{});
  }

  if constexpr (KSPLIT) {
    // group 1 hands its state to group 0 (same wavefront slot: same query rows, and lane
    // for lane the same half of each row).  The barriers order every wavefront's last
    // tile reads before the writes, and the writes before the reads.
    constexpr int kRegs = kDT * 16;
    float* const xf = (float*)lds + (size_t)wave * (kRegs + 2) * 64;
    tile_barrier();
    if (kgrp == 1) {
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[dt][4 * q + e];
          *(f32x4_t*)(xf + ((dt * 4 + q) * 64 + lane) * 4) = v;
        }
      xf[kRegs * 64 + lane] = m_run;          // -inf when this half had no tile for the row
      xf[kRegs * 64 + 64 + lane] = l_run;
    }
    tile_barrier();
    if (kgrp == 1) return;
    const float m1 = xf[kRegs * 64 + lane];
    const float l1 = xf[kRegs * 64 + 64 + lane];
    const float mn = fmaxf(m_run, m1);        // m_run is finite: group 0 always has tile 0
    const float a0 = fast_exp2((m_run - mn) * c2);
    const float a1 = fast_exp2((m1 - mn) * c2);   // 0 when m1 = -inf
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t v = *(const f32x4_t*)(xf + ((dt * 4 + q) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[dt][4 * q + e] = acc[dt][4 * q + e] * a0 + v[e] * a1;
      }
    l_run = l_run * a0 + l1 * a1;
    m_run = mn;
    mc = mn * c2;
  }

  // --- epilogue: O = acc / l, lse = m + ln l, each written once.
  const float l = sum_halves(l_run);
  const float inv = 1.0f / l;
  if (SPLIT && p.splits > 1) {
    // partial result of this key range: O_s = acc / l (float32) and lse_s = m + ln l
    // (a single range is the whole result: written below as the fused form writes it)
    if (qrow < N) {
      const size_t r = ((size_t)split * p.BH + bh) * (size_t)N + qrow;
      float* orow = p.part_o + r * D;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = acc[dt][4 * g + e] * inv;
          // register r of block dt: 16-bit inputs column 32dt + 16(r>>3) + 8G + (r&7),
          // fp32 inputs column 32dt + 8(r>>2) + 4G + (r&3)
          const int col = k16 ? dt * 32 + 16 * (g >> 1) + 8 * G + 4 * (g & 1) : dt * 32 + 8 * g + 4 * G;
          *(f32x4_t*)(orow + col) = ov;
        }
      if (G == 0) p.part_lse[r] = (mc + __builtin_amdgcn_logf(l)) * kLn2;
    }
    return;
  }
  if (qrow < N) {
    T* orow = (T*)p.o + head + (size_t)qrow * D;
    if constexpr (k16) {
      // register r of block dt is column 32dt + 16(r>>3) + 8G + (r&7)
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          h8_t ov;
#pragma unroll
          for (int e = 0; e < 8; ++e) ov[e] = (T)(acc[dt][8 * hh + e] * inv);
          *(h8_t*)(orow + dt * 32 + 16 * hh + 8 * G) = ov;
        }
    } else {
      // register r of block dt is column 32dt + 8(r>>2) + 4G + (r&3)
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = acc[dt][4 * g + e] * inv;
          *(f32x4_t*)(orow + dt * 32 + 8 * g + 4 * G) = ov;
        }
    }
    if (G == 0) p.lse[(size_t)bh * N + qrow] = (mc + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const Params& p, hipStream_t stream) {
  hipLaunchKernelGGL((mha_fwd_kernel<T, D, CAUSAL>), dim3(p.total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// 16-bit inputs: grids of at most one workgroup per CU (256 CUs) with at least two key
// tiles run the key-half form, which puts twice the wavefronts on each CU (measured on
// 256-workgroup grids: 1.06-1.09x at d = 128, 1.15-1.23x causal).  Larger grids keep the
// 4-wavefront form: at 512 workgroups and d = 64 (two per CU) the two forms were level
// (0.99-1.01x), the merge costing what the extra wavefronts gain.
template <typename T, int D, bool CAUSAL>
hipError_t launch16(const Params& p, hipStream_t stream) {
  constexpr int kCUs = 256;
  if (p.total <= kCUs && p.N > tile_keys<T, D, false>()) {
    hipLaunchKernelGGL((mha_fwd_kernel<T, D, CAUSAL, false, false, true>), dim3(p.total), dim3(2 * kThreads), 0,
                       stream, p);
    return hipGetLastError();
  }
  return launch<T, D, CAUSAL>(p, stream);
}

// Merge of the split-KV partial results (the cross-partition reduction of split-KV
// decoding): for one query row with partials (O_s, lse_s), s = 0..S-1,
//   lse = M + ln L,  M = max_s lse_s,  L = sum_s exp(lse_s - M),
//   O   = sum_s w_s * O_s,  w_s = exp(lse_s - M) / L.
// One workgroup of kMergeThreads per row.  M and L are block reductions over the splits
// (in-wavefront butterflies, then the 4 wavefront results through LDS); the weights go to
// LDS.  For O the threads form kGroups groups of D/4: thread (g, c) reads 4 columns of
// the partials s = g, g + kGroups, ... (16-byte loads, several in flight), and the
// groups' sums are added through LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeLdsWeights = 2048;

__device__ __forceinline__ float block_reduce(float x, float* red, bool is_max) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float y = __shfl_xor(x, off);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();   // red is written again by the next reduction
  return r;
}

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void mha_merge_kernel(Params p) {
  constexpr int kCols = D / 4;                       // threads per partial row (4 columns each)
  constexpr int kGroups = kMergeThreads / kCols;     // partial rows read side by side
  __shared__ float red[kMergeThreads / 64];
  __shared__ float wts[kMergeLdsWeights];
  __shared__ f32x4_t sums[kGroups][kCols];
  const size_t row = blockIdx.x;                      // (b*H + h) * N + query row
  const size_t stride = (size_t)p.BH * (size_t)p.N;   // between splits
  const int t = threadIdx.x;
  int splits = p.splits;
  if (p.seq_lens != nullptr) {
    // paged: only the key ranges below this sequence's key count were written
    const int b = (int)(row / p.N) / p.H;
    const int len = min(max(p.seq_lens[b], 0), p.max_blocks << p.bs_log2);
    splits = (len + p.chunk - 1) / p.chunk;
    if (splits == 0) {
      // no keys: the empty sum gives O = 0 and lse = log 0 = -inf
      for (int c = t; c < D; c += kMergeThreads) ((T*)p.o)[row * D + c] = (T)0.f;
      if (t == 0) p.lse[row] = -__builtin_inff();
      return;
    }
  }
  float m = -__builtin_inff();
  for (int s = t; s < splits; s += kMergeThreads) m = fmaxf(m, p.part_lse[s * stride + row]);
  const float M = block_reduce(m, red, true);
  float sum = 0.f;
  for (int s = t; s < splits; s += kMergeThreads) {
    const float e = __builtin_amdgcn_exp2f((p.part_lse[s * stride + row] - M) * kLog2e);
    sum += e;
    if (s < kMergeLdsWeights) wts[s] = e;
  }
  const float L = block_reduce(sum, red, false);     // its barrier also orders the wts writes
  const int c = t % kCols, g = t / kCols;
  const float* po = p.part_o + row * D + 4 * c;
  f32x4_t acc = {};
#pragma unroll 4
  for (int s = g; s < splits; s += kGroups) {
    const float w = s < kMergeLdsWeights ? wts[s]
                                         : __builtin_amdgcn_exp2f((p.part_lse[s * stride + row] - M) * kLog2e);
    acc += w * *(const f32x4_t*)(po + (size_t)s * stride * D);
  }
  sums[g][c] = acc;
  __syncthreads();
  if (t < kCols) {
    f32x4_t o = sums[0][t];
#pragma unroll
    for (int q = 1; q < kGroups; ++q) o += sums[q][t];
    const float invL = 1.0f / L;
#pragma unroll
    for (int e = 0; e < 4; ++e) ((T*)p.o)[row * D + 4 * t + e] = (T)(o[e] * invL);
  }
  if (t == 0) p.lse[row] = M + __builtin_amdgcn_logf(L) * kLn2;
}

template <typename T, int D, bool PAGED = false>
hipError_t launch_split(const Params& p, hipStream_t stream) {
  hipLaunchKernelGGL((mha_fwd_kernel<T, D, false, true, PAGED>), dim3(p.total), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;   // one range: the kernel wrote O and lse
  hipLaunchKernelGGL((mha_merge_kernel<T, D>), dim3(p.BH * p.N), dim3(kMergeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Static scratch of the no-allocation split-KV entry point: the float32 partial results
// (O then LSE of every split) of a call, in place of a caller workspace.  Each GPU holds
// its own copy at its own address; host code must use that address, never the array's
// name (which on the host only stands for the symbol).
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

int fwd_query_block(int) { return kBM; }

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int N, int d, int causal, float scale, int dtype, hipStream_t stream) {
  Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.N = N;
  p.nqb = (N + kBM - 1) / kBM;
  p.total = p.nqb * B * H;
  p.qmul = scale > 0.f ? 1.f : (scale < 0.f ? -1.f : 0.f);
  p.scale2 = (scale != 0.f ? fabsf(scale) : 1.f) * kLog2e;
  if (dtype == 1) {
    if (d == 64) return causal ? launch16<__bf16, 64, true>(p, stream) : launch16<__bf16, 64, false>(p, stream);
    return causal ? launch16<__bf16, 128, true>(p, stream) : launch16<__bf16, 128, false>(p, stream);
  }
  if (dtype == 2) {
    if (d == 64) return causal ? launch16<_Float16, 64, true>(p, stream) : launch16<_Float16, 64, false>(p, stream);
    return causal ? launch16<_Float16, 128, true>(p, stream) : launch16<_Float16, 128, false>(p, stream);
  }
  if (d == 64) return causal ? launch<float, 64, true>(p, stream) : launch<float, 64, false>(p, stream);
  return causal ? launch<float, 128, true>(p, stream) : launch<float, 128, false>(p, stream);
}

hipError_t launch_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                              int Nq, int Nk, int d, float scale, int dtype, int splits, int chunk,
                              float* part_o, float* part_lse, hipStream_t stream) {
  Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.N = Nq;
  p.nqb = (Nq + kBM - 1) / kBM;
  p.Nk = Nk;
  p.chunk = chunk;
  p.splits = splits;
  p.BH = B * H;
  p.part_o = part_o;
  p.part_lse = part_lse;
  p.total = p.nqb * p.BH * splits;
  p.qmul = scale > 0.f ? 1.f : (scale < 0.f ? -1.f : 0.f);
  p.scale2 = (scale != 0.f ? fabsf(scale) : 1.f) * kLog2e;
  if (dtype == 1) return d == 64 ? launch_split<__bf16, 64>(p, stream) : launch_split<__bf16, 128>(p, stream);
  if (dtype == 2) return d == 64 ? launch_split<_Float16, 64>(p, stream) : launch_split<_Float16, 128>(p, stream);
  return d == 64 ? launch_split<float, 64>(p, stream) : launch_split<float, 128>(p, stream);
}

hipError_t launch_fwd_paged(const void* q, const void* k_pool, const void* v_pool, const int* block_table,
                            const int* seq_lens, void* o, float* lse, int B, int H, int Nq, int d, float scale,
                            int dtype, int num_blocks, int bs_log2, int max_blocks, int splits, int chunk,
                            float* part_o, float* part_lse, hipStream_t stream) {
  Params p;
  p.q = q;
  p.k = k_pool;
  p.v = v_pool;
  p.o = o;
  p.lse = lse;
  p.N = Nq;
  p.nqb = (Nq + kBM - 1) / kBM;
  p.Nk = max_blocks << bs_log2;
  p.chunk = chunk;
  p.splits = splits;
  p.BH = B * H;
  p.part_o = part_o;
  p.part_lse = part_lse;
  p.total = p.nqb * p.BH * splits;
  p.qmul = scale > 0.f ? 1.f : (scale < 0.f ? -1.f : 0.f);
  p.scale2 = (scale != 0.f ? fabsf(scale) : 1.f) * kLog2e;
  p.H = H;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.max_blocks = max_blocks;
  p.num_blocks = num_blocks;
  p.bs_log2 = bs_log2;
  if (dtype == 1)
    return d == 64 ? launch_split<__bf16, 64, true>(p, stream) : launch_split<__bf16, 128, true>(p, stream);
  if (dtype == 2)
    return d == 64 ? launch_split<_Float16, 64, true>(p, stream) : launch_split<_Float16, 128, true>(p, stream);
  return d == 64 ? launch_split<float, 64, true>(p, stream) : launch_split<float, 128, true>(p, stream);
}

}  // namespace mha_impl
