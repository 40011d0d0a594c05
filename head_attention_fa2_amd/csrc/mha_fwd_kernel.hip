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
//  * A workgroup of 4 wavefronts owns 128 query rows, 32 per wavefront; two
//    workgroups (8 wavefronts, 2 per SIMD) share a CU.
//  * Both contractions are v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2_f32).
//    The scores are formed transposed, S^T = K.Q^T, so that lanes n and n+32 own ONE
//    query row: row max / row sum are in-lane reductions plus one v_permlane32_swap.  Output likewise is O^T = V^T.P^T, so the per-row rescale and
//    1/l are in-lane multiplies.
//  * K rows enter the first product in an order that swaps bits 2 and 3 of the row
//    index inside each 32-row slab; the fp32 accumulator of S^T is then, register for
//    register, the bf16 B operand P^T of the second product, so P needs no shuffle.
//  * K/V rows are copied HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging) into
//    rings of four 32-key slab buffers each; every 64 keys one barrier, after which the
//    next 64 keys of K (one slab further ahead) and of V are copied.
//    LDS rows are XOR-swizzled in 16-byte chunks so that the MFMA operand reads of
//    K (ds_read_b128) and of V^T (ds_read_b64_tr_b16, the gfx950 transposing LDS read)
//    are free of bank conflicts.
//  * Software pipeline inside each wavefront over 32-key slabs (the matrix cores run
//    while the vector units work on independent data): while the MFMAs of
//    S_{s+1} = K_{s+1}.Q^T issue, the VALU evaluates exp2, the bf16 conversion and the
//    row sums of slab s; while the MFMAs of O += V_s^T.P_s^T issue, the VALU masks slab
//    s+1, takes its row max and forms the exponent arguments.
//  * exp is evaluated as exp2 with the scale folded into one FMA (log2(e) prescale, as
//    the "Long Softmax" puzzle recommends).  The output rescale is lazy: the running max
//    used as exponent offset only moves when the true max exceeds it by more than 2^8
//    in the exponent; O / l and m + ln l are exact for whichever offset was used.
//  * Causal: key tiles entirely after a wavefront's rows are skipped, only tiles that
//    cross the diagonal (or the ragged end of the sequence) evaluate the mask, and
//    heavy (late) query blocks are scheduled first.  Workgroup ids are remapped so that
//    all query blocks of a head run on the same XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mha_launch.h"
#include "mha_layout.h"

// copy_to_lds sets m0 itself right before each copy and nothing else in these kernels
// reads m0, so declaring it clobbered is sound (the build passes -Wno-inline-asm for
// the backend's generic warning about clobbering a reserved register).

namespace mha_impl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kBN = 64;                  // keys copied per barrier (two 32-key slabs)
constexpr int kSlab = 32;                // keys per pipeline step
constexpr int kWaves = 4;                // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;     // lazy-rescale threshold, in log2 units

// 32-row query groups per wavefront, rows per wavefront, rows per workgroup.
template <typename T>
struct Rows {
  static constexpr int kQG = 1;
  static constexpr int kQW = 32 * kQG;
  static constexpr int kBM = kQW * kWaves;
};

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;          // sequence length
  int nqb;        // query blocks per head
  int total;      // workgroups
  float qmul;     // sign(scale): Q is multiplied by it on load (1, -1 or 0)
  float scale2;   // |scale| * log2(e), or log2(e) when scale == 0
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

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One 16-byte-per-lane copy HBM -> LDS (global_load_lds_dwordx4): lane l reads
// sbase + voff and the data lands at LDS address lds + 16*l.  Issued as inline asm so
// that the compiler does not track it: the only waits on these copies are the explicit
// vmcnt waits of the tile pipeline, which order them against the LDS reads.
__device__ __forceinline__ void copy_to_lds(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wavefront are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier for the LDS tile pipeline.  __syncthreads() would also wait for
// every outstanding global load, including the prefetch of the next tile; here each
// wavefront has already waited (vmcnt) for the loads of the tile about to be read, and
// its LDS reads of the previous tile were consumed before it arrives, so only the
// execution barrier is needed.  The empty asm statements keep the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void tile_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------- kernel
// Two workgroups (8 wavefronts, 2 per SIMD) per CU when the slab rings fit twice in the
// 160 KiB of LDS; fp32 with d = 128 needs 128 KiB and runs one workgroup per CU.
template <typename T, int D>
constexpr int min_waves_per_eu() { return 8 * kSlab * D * (int)sizeof(T) <= 80 * 1024 ? 2 : 1; }

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(min_waves_per_eu<T, D>())))
void mha_fwd_kernel(Params p) {
  constexpr bool kBF16 = sizeof(T) == 2;
  constexpr int kQW = Rows<T>::kQW;             // 32 query rows per wavefront
  constexpr int kBM = Rows<T>::kBM;
  constexpr int RB = D * (int)sizeof(T);        // bytes per K/V row
  constexpr int R = RB / 16;                     // 16-byte chunks per row
  constexpr int kSlabBytes = kSlab * RB;
  constexpr int kLoads = kBN * R / kThreads;     // 16-byte copies per thread per 64 rows
  static_assert(kLoads * kThreads == kBN * R && kLoads % 2 == 0, "copies must split evenly");
  constexpr int kDT = D / 32;                    // 32-wide output column blocks
  constexpr int kQF = kBF16 ? D / 16 : D / 8;    // Q operand fragments

  // Rings of four 32-key slab buffers: [K slabs 0..3][V slabs 0..3].  Slab s of the
  // sequence lives in buffer s % 4.
  __shared__ __attribute__((aligned(1024))) char smem[8 * kSlabBytes];
  auto kslab = [&](int b) { return smem + b * kSlabBytes; };
  auto vslab = [&](int b) { return smem + (4 + b) * kSlabBytes; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;      // query column (and K row slot) within the wavefront
  const int G = lane >> 5;      // lane half

  // --- workgroup -> (head, query block).  Consecutive workgroup ids go to different
  // XCDs, so renumber: the k-th workgroup dispatched to XCD x gets task x*T/8 + k, which
  // keeps every head's query blocks on one XCD.  Causal: latest (heaviest) blocks first.
  int id = blockIdx.x;
  if ((p.total & 7) == 0) id = (id & 7) * (p.total >> 3) + (id >> 3);
  const int bh = id / p.nqb;
  int qb = id - bh * p.nqb;
  if (CAUSAL) qb = p.nqb - 1 - qb;
  const int N = p.N;
  const int q0 = qb * kBM;
  const int qw = q0 + wave * kQW;               // first query row of this wavefront
  const int qrow = qw + n;                      // the query row this lane owns
  const size_t head = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Q = (const T*)p.q + head;
  const char* Kbase = (const char*)((const T*)p.k + head);
  const char* Vbase = (const char*)((const T*)p.v + head);

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int ntiles = (kv_end + kBN - 1) / kBN;  // 64-key copy steps of the workgroup
  // last slab with a key visible to some row of this wavefront (later slabs are skipped
  // by this wavefront; it still takes part in the cooperative copies)
  const int last_s = min((kv_end - 1) / kSlab, CAUSAL ? (qw + kQW - 1) / kSlab : 1 << 30);

  // --- copies: 64 consecutive K or V rows starting at row r0, split into two slab
  // buffers.  Copy j of a thread fills LDS bytes [(j*kWaves + wave)*1024, +1024) of the
  // 64-row span: copies j < kLoads/2 land in the first slab, the rest in the second.
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
  const unsigned ld_off0 = (unsigned)(ld_row[0] * RB + ld_chunk[0] * 16);
  // rows [r0, r0 + 32 * halves) -> slab buffers (a, b); halves = 1 copies only the first
  auto issue_span = [&](const char* base, int r0, char* a, char* b, int halves)
      __attribute__((always_inline)) {
    const char* g = base + (size_t)r0 * RB;
    const bool whole = r0 + kSlab * halves <= N;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      if (j >= kLoads / 2 && halves < 2) break;
      char* dst = (j < kLoads / 2 ? a : b - kSlabBytes) + (j * kWaves + wave) * 1024;
      unsigned off;
      if (whole) {
        off = mha_layout::loader_periodic<R>() ? ld_off0 + (unsigned)(j * kRowStep * RB)
                                               : (unsigned)(ld_row[j] * RB + ld_chunk[j] * 16);
      } else {
        // ragged end: rows past the end re-read row N-1 (finite, masked later)
        off = (unsigned)((min(r0 + ld_row[j], N - 1) - r0) * RB + ld_chunk[j] * 16);
      }
      copy_to_lds(g, off, lds_addr(dst));
    }
  };

  // --- Q operand, kept in registers for the whole loop ("Load Q" once).
  // bf16: lane (n, G) holds Q[qrow][16kc + 8G .. +7].  fp32: Q[qrow][8j + 4G .. +3].
  typedef typename std::conditional<kBF16, bf16x8_t, f32x4_t>::type qfrag_t;
  qfrag_t qf[kQF];
  {
    const bool valid = qrow < N;
    const T* qr = Q + (size_t)(valid ? qrow : 0) * D;
#pragma unroll
    for (int j = 0; j < kQF; ++j) {
      const int col = kBF16 ? 16 * j + 8 * G : 8 * j + 4 * G;
      qf[j] = *(const qfrag_t*)(qr + col);
      if (!valid) qf[j] = qfrag_t{};
      // scaled logit = scale * q.k = |scale| * (sign(scale) q).k; multiplying by 1, -1
      // or 0 is exact, so the row max below is always taken on the logit's own order.
#pragma unroll
      for (int e = 0; e < (int)(sizeof(qfrag_t) / sizeof(T)); ++e) qf[j][e] = (T)((float)qf[j][e] * p.qmul);
    }
  }

  // --- per-lane LDS offsets of the MFMA operands within a slab buffer.
  int offK[kQF];
#pragma unroll
  for (int j = 0; j < kQF; ++j) offK[j] = mha_layout::k_operand_off<R>(lane, j);
  int offV[kBF16 ? kDT : 1][2];
  if constexpr (kBF16) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) offV[dt][h] = mha_layout::v_operand_off<R>(lane, dt, h);
  }

  // --- running state of this lane's query row.
  f32x16_t acc[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) acc[dt] = f32x16_t{};
  float m_run = -__builtin_inff();   // exponent offset in raw score units
  float l_run = 0.f;                 // this lane's share of the row sum
  float alpha = 1.f;                 // pending rescale of O
  bool rescale = false;              // wavefront-uniform: alpha must be applied to O
  const float c2 = p.scale2;

  // S^T = K_s . Q^T for one 32-key slab; register r on lane half G is key
  // 16(r>>3) + 8G + (r&7) of the slab.
  auto qk = [&](const char* lk, f32x16_t& s) __attribute__((always_inline)) {
    s = f32x16_t{};
    if constexpr (kBF16) {
#pragma unroll
      for (int kc = 0; kc < kQF; ++kc) {
        const bf16x8_t kf = *(const bf16x8_t*)(lk + offK[kc]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kc], s, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kQF; ++j) {
        const f32x4_t kf = *(const f32x4_t*)(lk + offK[j]);
#pragma unroll
        for (int t = 0; t < 4; ++t) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[t], qf[j][t], s, 0, 0, 0);
      }
    }
  };

  // First half of the online softmax of slab si (the running max of the "Long Softmax"
  // puzzle): mask, row max, lazy rescale decision, and s <- c2 (s - m) in place.
  auto stats = [&](f32x16_t& s, int si, auto masked_tag) __attribute__((always_inline)) {
    if constexpr (decltype(masked_tag)::value) {
      const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = si * kSlab + 16 * (r >> 3) + 8 * G + (r & 7);
        if (key > lim) s[r] = -__builtin_inff();
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx);
    // move the exponent offset only when the max grew by more than 2^8 (or on the
    // first slab); decided for the whole wavefront
    const bool any_grow = __builtin_amdgcn_ballot_w64((m_new - m_run) * c2 > kRescaleLog2) != 0;
    const float m_use = any_grow ? (m_new == -__builtin_inff() ? 0.f : m_new) : m_run;
    alpha = any_grow ? fast_exp2((m_run - m_use) * c2) : 1.0f;   // 0 from -inf
    l_run *= alpha;
    m_run = m_use;
    rescale = any_grow;
    const float mc = (m_use == -__builtin_inff() ? 0.f : m_use) * c2;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(s[r], c2, -mc);
  };

  // Second half: p = exp2(s), the row sum (float32 p, so that ln l keeps full
  // precision even for rows that see few keys), and (bf16) the P^T operands of the
  // slab: operand hh holds keys 16hh + 8G + e on lane half G.
  auto expsum = [&](f32x16_t& s, bf16x8_t (&pf)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = fast_exp2(s[r]);
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) lsum += s[r];
    l_run += lsum;
    if constexpr (kBF16) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[hh][e] = (__bf16)s[8 * hh + e];
    }
  };

  // O <- alpha O when the exponent offset moved (rare).
  auto rescale_o = [&]() __attribute__((always_inline)) {
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) acc[dt] *= alpha;
    }
  };

  // O^T += V_s^T . P_s^T for one slab.
  auto pv = [&](const char* lv, const bf16x8_t (&pf)[2], const f32x16_t& s) __attribute__((always_inline)) {
    if constexpr (kBF16) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(lv + offV[dt][0] + hh * 16 * RB));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(lv + offV[dt][1] + hh * 16 * RB));
          const bf16x8_t vf =
              __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[hh], acc[dt], 0, 0, 0);
        }
    } else {
      // fp32: two keys per MFMA; B operand = p in register u, A operand on lane (m, G) =
      // V[key of register u on half G][32dt + m].
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int key = 16 * (u >> 3) + 8 * G + (u & 7);
          const int col = dt * 32 + n;
          const float vv = *(const float*)(lv + lds_off<R>(key, col >> 2) + (col & 3) * 4);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, s[u], acc[dt], 0, 0, 0);
        }
    }
  };

  auto slab_masked = [&](int si) __attribute__((always_inline)) {
    const int k0 = si * kSlab;
    return (k0 + kSlab > N) || (CAUSAL && k0 + kSlab - 1 > qw);
  };

  // MFMA / VALU interleave hints for the two regions of a step (bf16).
  constexpr int kMfmaQK = kQF;              // MFMAs of S_{s+1}
  constexpr int kMfmaPV = 2 * kDT;          // MFMAs of O += V_s^T P_s^T
  auto interleave_qk = [&]() __attribute__((always_inline)) {
    if constexpr (kBF16) {
      // K operands two MFMAs ahead; exp2 / sum / convert of slab s between the MFMAs
      constexpr int kValu = (16 + 16 + 8 + kMfmaQK - 1) / kMfmaQK;
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < kMfmaQK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
        if (i < kMfmaQK - 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  auto interleave_pv = [&]() __attribute__((always_inline)) {
    if constexpr (kBF16) {
      // V^T operands (two transposing reads each) two MFMAs ahead; mask / max /
      // exponent arguments of slab s+1 between the MFMAs
      constexpr int kValu = (8 + 16 + 10 + kMfmaPV - 1) / kMfmaPV;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < kMfmaPV; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
        if (i < kMfmaPV - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };

  // --- main loop over 32-key slabs.  Sub-step s of a wavefront:
  //   region A: MFMAs of S_{s+1} = K_{s+1}.Q^T  ||  exp2 / convert / row sum of slab s
  //   O rescale for slab s (rare)
  //   region C: MFMAs of O += V_s^T.P_s^T       ||  mask / max / exponent args of slab s+1
  // Step j = sub-steps 2j, 2j+1 reads K slabs 2j+1, 2j+2 and V slabs 2j, 2j+1, all
  // copied during step j-1 (or the prologue); after its barrier it copies K slabs 2j+3,
  // 2j+4 and V slabs 2j+2, 2j+3 into the ring buffers last read during step j-1.  Slab
  // scores ping-pong between two register sets by sub-step parity.
  f32x16_t sbuf[2];
  issue_span(Kbase, 0, kslab(0), kslab(1), 2);
  issue_span(Vbase, 0, vslab(0), vslab(1), 2);
  if (kv_end > kBN) issue_span(Kbase, kBN, kslab(2), nullptr, 1);
  wait_vmcnt<0>();
  tile_barrier();
  qk(kslab(0), sbuf[0]);
  if (slab_masked(0)) stats(sbuf[0], 0, std::true_type{});
  else stats(sbuf[0], 0, std::false_type{});
  rescale = false;                          // O is still zero

  // sub-step si (parity P): K buffer kb holds slab si+1, V buffer vb holds slab si
  auto substep = [&](int si, auto par_tag, auto kb_tag, auto vb_tag) __attribute__((always_inline)) {
    constexpr int par = decltype(par_tag)::value;
    constexpr int kb = decltype(kb_tag)::value;
    constexpr int vb = decltype(vb_tag)::value;
    f32x16_t& s_cur = sbuf[par];
    f32x16_t& s_next = sbuf[par ^ 1];
    bf16x8_t pf[2];
    if (si + 1 <= last_s) {
      qk(kslab(kb), s_next);
      expsum(s_cur, pf);
      interleave_qk();
      __builtin_amdgcn_sched_barrier(0);
      rescale_o();
      __builtin_amdgcn_sched_barrier(0);
      if (slab_masked(si + 1)) {
        pv(vslab(vb), pf, s_cur);
        stats(s_next, si + 1, std::true_type{});
        interleave_pv();
      } else {
        pv(vslab(vb), pf, s_cur);
        stats(s_next, si + 1, std::false_type{});
        interleave_pv();
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
      if (si <= last_s) {
        expsum(s_cur, pf);
        __builtin_amdgcn_sched_barrier(0);
        rescale_o();
        __builtin_amdgcn_sched_barrier(0);
        pv(vslab(vb), pf, s_cur);
      }
      // no later slab for this wavefront: define the next scores so that no stale
      // register set stays live across sub-steps
      s_next = f32x16_t{};
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto step = [&](int j, auto jpar_tag) __attribute__((always_inline)) {
    constexpr int jp = decltype(jpar_tag)::value;          // j & 1
    wait_vmcnt<0>();
    tile_barrier();
    // copies for step j+1: K rows [64j+96, 64j+160) -> K slabs 2j+3, 2j+4 and V rows
    // [64j+64, 64j+128) -> V slabs 2j+2, 2j+3 (buffer = slab % 4)
    const int k_r0 = kBN * j + 3 * kSlab;
    if (k_r0 < kv_end)
      issue_span(Kbase, k_r0, kslab(jp ? 1 : 3), kslab(jp ? 2 : 0), k_r0 + kSlab < kv_end ? 2 : 1);
    const int v_r0 = kBN * (j + 1);
    if (v_r0 < kv_end) issue_span(Vbase, v_r0, vslab(jp ? 0 : 2), vslab(jp ? 1 : 3), 2);
    // sub-steps 2j (K slab 2j+1, V slab 2j) and 2j+1 (K slab 2j+2, V slab 2j+1)
    if constexpr (jp == 0) {
      substep(2 * j, I0{}, I1{}, I0{});
      substep(2 * j + 1, I1{}, I2{}, I1{});
    } else {
      substep(2 * j, I0{}, I3{}, I2{});
      substep(2 * j + 1, I1{}, I0{}, I3{});
    }
  };
  for (int j = 0; j < ntiles; j += 2) {
    step(j, I0{});
    if (j + 1 < ntiles) step(j + 1, I1{});
  }

  // --- epilogue: O = acc / l, lse = m + ln l, each written once.
  const float l = sum_halves(l_run);
  const float inv = 1.0f / l;
  if (qrow < N) {
    T* orow = (T*)p.o + head + (size_t)qrow * D;
    if constexpr (kBF16) {
      // register r of block dt is column 32dt + 16(r>>3) + 8G + (r&7)
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8_t ov;
#pragma unroll
          for (int e = 0; e < 8; ++e) ov[e] = (__bf16)(acc[dt][8 * hh + e] * inv);
          *(bf16x8_t*)(orow + dt * 32 + 16 * hh + 8 * G) = ov;
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
    if (G == 0) p.lse[(size_t)bh * N + qrow] = (m_run * c2 + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const Params& p, hipStream_t stream) {
  hipLaunchKernelGGL((mha_fwd_kernel<T, D, CAUSAL>), dim3(p.total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int fwd_query_block(int is_bf16) { return is_bf16 ? Rows<__bf16>::kBM : Rows<float>::kBM; }

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int N, int d, int causal, float scale, int is_bf16, hipStream_t stream) {
  Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.N = N;
  const int bm = fwd_query_block(is_bf16);
  p.nqb = (N + bm - 1) / bm;
  p.total = p.nqb * B * H;
  p.qmul = scale > 0.f ? 1.f : (scale < 0.f ? -1.f : 0.f);
  p.scale2 = (scale != 0.f ? fabsf(scale) : 1.f) * kLog2e;
  if (is_bf16) {
    if (d == 64) return causal ? launch<__bf16, 64, true>(p, stream) : launch<__bf16, 64, false>(p, stream);
    return causal ? launch<__bf16, 128, true>(p, stream) : launch<__bf16, 128, false>(p, stream);
  }
  if (d == 64) return causal ? launch<float, 64, true>(p, stream) : launch<float, 64, false>(p, stream);
  return causal ? launch<float, 128, true>(p, stream) : launch<float, 128, false>(p, stream);
}

}  // namespace mha_impl
