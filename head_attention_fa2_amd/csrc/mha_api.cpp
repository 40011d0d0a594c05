// C ABI of libmha.so: argument validation on the host, then one kernel launch.
// The entry points and their contracts are declared in include/mha.h.
#include "mha.h"

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "mha_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mha_status validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    int B, int H, int N, int d, int causal, float scale, mha_dtype dtype) {
  if (!q || !k || !v || !o || !lse) return MHA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return MHA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MHA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_F32 && dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_F16) return MHA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MHA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return MHA_ERR_UNSUPPORTED;
  const int64_t bm = mha_impl::fwd_query_block((int)dtype);
  const int64_t blocks = ((int64_t)N + bm - 1) / bm * (int64_t)B * (int64_t)H;
  if (blocks > INT32_MAX) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

// Split-KV partition: `splits` requested (0 = automatic), resolved to key ranges of
// `chunk` keys (a multiple of the 64-key tile) and the number of non-empty ranges.
// Automatic: enough ranges for about 512 workgroups (two per CU of the MI355X), each of
// at least 512 keys.
struct Partition {
  int splits;
  int chunk;
};
Partition partition(int B, int H, int Nq, int Nk, int splits) {
  const int64_t bm = mha_impl::fwd_query_block(1);
  const int64_t blocks = ((int64_t)Nq + bm - 1) / bm * (int64_t)B * (int64_t)H;
  int64_t s = splits;
  if (s <= 0) {
    s = (512 + blocks - 1) / blocks;
    const int64_t cap = ((int64_t)Nk + 511) / 512;
    if (s > cap) s = cap;
  }
  const int64_t tiles = ((int64_t)Nk + 63) / 64;
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  const int64_t chunk = (tiles + s - 1) / s * 64;
  return Partition{(int)(((int64_t)Nk + chunk - 1) / chunk), (int)chunk};
}

// Paged: the automatic choice is the split-KV one over the longest possible sequence
// (max_blocks * block_size keys).  Measured on the paged decoding workloads (lengths
// 256..16384, 512 and more heads x sequences), one range per sequence beat 2, 4, 8 and 16:
// short sequences finish early and the long ones then get more of the bandwidth.
Partition partition_paged(int B, int H, int Nq, int max_keys, int splits) {
  return partition(B, H, Nq, max_keys, splits);
}

size_t workspace_bytes(int B, int H, int Nq, int d, int splits) {
  return (size_t)splits * (size_t)B * (size_t)H * (size_t)Nq * ((size_t)d + 1) * sizeof(float);
}

// Split-KV checks of everything but the workspace.
mha_status validate_splitkv_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 int B, int H, int Nq, int Nk, int d, float scale, mha_dtype dtype, int splits) {
  if (!q || !k || !v || !o || !lse) return MHA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || splits < 0) return MHA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_F32 && dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_F16) return MHA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MHA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return MHA_ERR_UNSUPPORTED;
  const Partition pt = partition(B, H, Nq, Nk, splits);
  const int64_t bm = mha_impl::fwd_query_block((int)dtype);
  const int64_t blocks = ((int64_t)Nq + bm - 1) / bm * (int64_t)B * (int64_t)H * pt.splits;
  if (blocks > INT32_MAX || (int64_t)B * H * Nq > INT32_MAX) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

mha_status validate_splitkv(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            int B, int H, int Nq, int Nk, int d, float scale, mha_dtype dtype, int splits,
                            const void* workspace, size_t ws_bytes) {
  if (!workspace) return MHA_ERR_INVALID_ARG;
  const mha_status st = validate_splitkv_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, dtype, splits);
  if (st != MHA_OK) return st;
  if (!aligned16(workspace)) return MHA_ERR_UNSUPPORTED;
  if (ws_bytes < workspace_bytes(B, H, Nq, d, partition(B, H, Nq, Nk, splits).splits)) return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

// Paged K/V: block size a power of two in [16, 65536]; the key range of every sequence
// is at most max_blocks * block_size keys, which sizes the partition and workspace.
int block_size_log2(int block_size) {
  if (block_size < 16 || block_size > 65536 || (block_size & (block_size - 1)) != 0) return -1;
  int l = 0;
  while ((1 << l) < block_size) ++l;
  return l;
}

mha_status validate_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, const void* o, const float* lse, int B, int H, int Nq, int d,
                          int num_blocks, int block_size, int max_blocks, float scale, mha_dtype dtype, int splits,
                          const void* workspace, size_t ws_bytes) {
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o || !lse || !workspace)
    return MHA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Nq < 1 || num_blocks < 1 || max_blocks < 1 || splits < 0) return MHA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_F32 && dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_F16) return MHA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MHA_ERR_UNSUPPORTED;
  if (block_size_log2(block_size) < 0) return MHA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace) || (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0)
    return MHA_ERR_UNSUPPORTED;
  const int64_t max_keys = (int64_t)max_blocks * block_size;
  if (max_keys > (int64_t)1 << 30) return MHA_ERR_UNSUPPORTED;
  const Partition pt = partition_paged(B, H, Nq, (int)max_keys, splits);
  if (ws_bytes < workspace_bytes(B, H, Nq, d, pt.splits)) return MHA_ERR_INVALID_ARG;
  const int64_t bm = mha_impl::fwd_query_block((int)dtype);
  const int64_t blocks = ((int64_t)Nq + bm - 1) / bm * (int64_t)B * (int64_t)H * pt.splits;
  if (blocks > INT32_MAX || (int64_t)B * H * Nq > INT32_MAX || (int64_t)B * max_blocks > INT32_MAX)
    return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

mha_status validate_gemm(const void* a, const void* b, const void* c, int M, int N, int K, mha_dtype dtype) {
  if (!a || !b || !c) return MHA_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_F32 && dtype != MHA_DTYPE_BF16 && dtype != MHA_DTYPE_F16) return MHA_ERR_INVALID_ARG;
  if (dtype == MHA_DTYPE_F32) return MHA_ERR_UNSUPPORTED;
  if (N % 8 != 0 || K % 8 != 0) return MHA_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return MHA_ERR_UNSUPPORTED;
  // 32-bit byte offsets inside A and B; the tile count (at the smallest tiling, 128 x 64)
  // fits the grid
  if ((int64_t)M * K * 2 > UINT32_MAX || (int64_t)K * N * 2 > UINT32_MAX) return MHA_ERR_UNSUPPORTED;
  if (((int64_t)M + 127) / 128 * (((int64_t)N + 63) / 64) > INT32_MAX) return MHA_ERR_UNSUPPORTED;
  return MHA_OK;
}

// Split-K GEMM partition: `splits` requested (0 = automatic), resolved to ranges of
// `kchunk` (a multiple of the 64-wide k-step) and the number of non-empty ranges.
// Automatic: a power of two, the largest that keeps the grid within about 512
// workgroups over the 128 x 128 tiles and every range at least 4 k-steps (measured on
// the memory-bound shapes: the power of two beat its neighbours, e.g. 4 splits at 4.9
// TB/s against 5 at 3.6 for M = 16, N = 14336, K = 4096).
Partition gemm_splitk_partition(int M, int N, int K, int splits) {
  const int64_t tiles = ((int64_t)M + 127) / 128 * (((int64_t)N + 127) / 128);
  const int64_t steps = ((int64_t)K + 63) / 64;
  int64_t s = splits;
  if (s <= 0) {
    int64_t want = (512 + tiles - 1) / tiles;
    const int64_t cap = (steps + 3) / 4;
    if (want > cap) want = cap;
    s = 1;
    while (s * 2 <= want) s *= 2;
  }
  if (s > steps) s = steps;
  if (s < 1) s = 1;
  const int64_t kchunk = (steps + s - 1) / s * 64;
  return Partition{(int)(((int64_t)K + kchunk - 1) / kchunk), (int)kchunk};
}

size_t gemm_splitk_workspace_bytes(int M, int N, int splits) {
  return (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
}

mha_status validate_gemm_splitk(const void* a, const void* b, const void* c, int M, int N, int K, mha_dtype dtype,
                                int splits, const void* workspace, size_t ws_bytes) {
  const mha_status st = validate_gemm(a, b, c, M, N, K, dtype);
  if (st != MHA_OK) return st;
  if (!workspace || splits < 0) return MHA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return MHA_ERR_UNSUPPORTED;
  const Partition pt = gemm_splitk_partition(M, N, K, splits);
  if ((int64_t)M * N > INT32_MAX || ((int64_t)M + 127) / 128 * (((int64_t)N + 127) / 128) * pt.splits > INT32_MAX)
    return MHA_ERR_UNSUPPORTED;
  if (ws_bytes < gemm_splitk_workspace_bytes(M, N, pt.splits)) return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

}  // namespace

extern "C" {

mha_status mha_fwd_validate(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, int B, int H, int N, int d, int causal, float scale,
                            mha_dtype dtype) {
  return validate(q, k, v, o, lse, B, H, N, d, causal, scale, dtype);
}

mha_status mha_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, int causal, float scale, mha_dtype dtype, hipStream_t stream) {
  const mha_status st = validate(q, k, v, o, lse, B, H, N, d, causal, scale, dtype);
  if (st != MHA_OK) return st;
  const hipError_t e = mha_impl::launch_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, (int)dtype,
                                            stream);
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

int mha_fwd_splitkv_splits(int B, int H, int Nq, int Nk, int splits) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || splits < 0) return 0;
  return partition(B, H, Nq, Nk, splits).splits;
}

size_t mha_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d, int splits) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || splits < 0 || d < 1) return 0;
  return workspace_bytes(B, H, Nq, d, partition(B, H, Nq, Nk, splits).splits);
}

mha_status mha_fwd_splitkv_validate(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                                    mha_dtype dtype, int splits, const void* workspace,
                                    size_t workspace_bytes) {
  return validate_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, dtype, splits, workspace, workspace_bytes);
}

mha_status mha_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                           int Nq, int Nk, int d, float scale, mha_dtype dtype, int splits, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  const mha_status st =
      validate_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, dtype, splits, workspace, workspace_bytes);
  if (st != MHA_OK) return st;
  const Partition pt = partition(B, H, Nq, Nk, splits);
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = part_o + (size_t)pt.splits * B * H * Nq * d;
  const hipError_t e = mha_impl::launch_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, (int)dtype, pt.splits,
                                                    pt.chunk, part_o, part_lse, stream);
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

mha_status mha_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                   int Nq, int Nk, int d, float scale, mha_dtype dtype, int splits,
                                   hipStream_t stream) {
  const mha_status st = validate_splitkv_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, dtype, splits);
  if (st != MHA_OK) return st;
  const Partition pt = partition(B, H, Nq, Nk, splits);
  if (workspace_bytes(B, H, Nq, d, pt.splits) > mha_impl::scratch_bytes()) return MHA_ERR_SCRATCH;
  void* scratch = nullptr;
  if (mha_impl::scratch_address(&scratch) != hipSuccess) return MHA_ERR_HIP;
  float* part_o = static_cast<float*>(scratch);
  float* part_lse = part_o + (size_t)pt.splits * B * H * Nq * d;
  const hipError_t e = mha_impl::launch_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, (int)dtype, pt.splits,
                                                    pt.chunk, part_o, part_lse, stream);
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

mha_status mha_fwd_paged_validate(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* seq_lens, const void* o,
                                  const float* lse, int B, int H, int Nq, int d, int num_blocks, int block_size,
                                  int max_blocks, float scale, mha_dtype dtype, int splits, const void* workspace,
                                  size_t workspace_bytes) {
  return validate_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H, Nq, d, num_blocks, block_size,
                        max_blocks, scale, dtype, splits, workspace, workspace_bytes);
}

mha_status mha_fwd_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                         const int32_t* seq_lens, void* o, float* lse, int B, int H, int Nq, int d, int num_blocks,
                         int block_size, int max_blocks, float scale, mha_dtype dtype, int splits, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  const mha_status st = validate_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H, Nq, d, num_blocks,
                                       block_size, max_blocks, scale, dtype, splits, workspace, workspace_bytes);
  if (st != MHA_OK) return st;
  const Partition pt = partition_paged(B, H, Nq, max_blocks * block_size, splits);
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = part_o + (size_t)pt.splits * B * H * Nq * d;
  const hipError_t e = mha_impl::launch_fwd_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H, Nq, d,
                                                  scale, (int)dtype, num_blocks, block_size_log2(block_size),
                                                  max_blocks, pt.splits, pt.chunk, part_o, part_lse,
                                                  stream);
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

int mha_fwd_paged_splits(int B, int H, int Nq, int block_size, int max_blocks, int splits) {
  if (B < 1 || H < 1 || Nq < 1 || max_blocks < 1 || splits < 0 || block_size_log2(block_size) < 0) return 0;
  if ((int64_t)max_blocks * block_size > (int64_t)1 << 30) return 0;
  return partition_paged(B, H, Nq, max_blocks * block_size, splits).splits;
}

size_t mha_fwd_paged_workspace_size(int B, int H, int Nq, int d, int block_size, int max_blocks, int splits) {
  const int s = mha_fwd_paged_splits(B, H, Nq, block_size, max_blocks, splits);
  if (s == 0 || d < 1) return 0;
  return workspace_bytes(B, H, Nq, d, s);
}

double mha_fwd_paged_bytes(int B, int H, int Nq, long long total_keys, int d, mha_dtype dtype) {
  const double elem = dtype == MHA_DTYPE_F32 ? 4.0 : 2.0;
  return (2.0 * B * Nq + 2.0 * (double)total_keys) * H * (double)d * elem + 4.0 * B * H * (double)Nq;
}

mha_status mha_gemm_validate(const void* a, const void* b, const void* c, int M, int N, int K, mha_dtype dtype) {
  return validate_gemm(a, b, c, M, N, K, dtype);
}

mha_status mha_gemm(const void* a, const void* b, void* c, int M, int N, int K, mha_dtype dtype, hipStream_t stream) {
  const mha_status st = validate_gemm(a, b, c, M, N, K, dtype);
  if (st != MHA_OK) return st;
  const hipError_t e = mha_impl::launch_gemm(a, b, c, M, N, K, (int)dtype, stream);
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

int mha_gemm_splitk_splits(int M, int N, int K, int splits) {
  if (M < 1 || N < 1 || K < 1 || splits < 0) return 0;
  return gemm_splitk_partition(M, N, K, splits).splits;
}

size_t mha_gemm_splitk_workspace_size(int M, int N, int K, int splits) {
  if (M < 1 || N < 1 || K < 1 || splits < 0) return 0;
  return gemm_splitk_workspace_bytes(M, N, gemm_splitk_partition(M, N, K, splits).splits);
}

mha_status mha_gemm_splitk_validate(const void* a, const void* b, const void* c, int M, int N, int K,
                                    mha_dtype dtype, int splits, const void* workspace, size_t workspace_bytes) {
  return validate_gemm_splitk(a, b, c, M, N, K, dtype, splits, workspace, workspace_bytes);
}

mha_status mha_gemm_splitk(const void* a, const void* b, void* c, int M, int N, int K, mha_dtype dtype, int splits,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const mha_status st = validate_gemm_splitk(a, b, c, M, N, K, dtype, splits, workspace, workspace_bytes);
  if (st != MHA_OK) return st;
  const Partition pt = gemm_splitk_partition(M, N, K, splits);
  const hipError_t e = mha_impl::launch_gemm_splitk(a, b, c, M, N, K, (int)dtype, pt.splits, pt.chunk,
                                                    static_cast<float*>(workspace), stream);
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

double mha_gemm_flops(int M, int N, int K) { return 2.0 * M * (double)N * (double)K; }

double mha_gemm_bytes(int M, int N, int K, mha_dtype dtype) {
  const double elem = dtype == MHA_DTYPE_F32 ? 4.0 : 2.0;
  return ((double)M * K + (double)K * N + (double)M * N) * elem;
}

double mha_fwd_splitkv_bytes(int B, int H, int Nq, int Nk, int d, mha_dtype dtype) {
  const double elem = dtype == MHA_DTYPE_F32 ? 4.0 : 2.0;
  return (2.0 * Nq + 2.0 * Nk) * B * H * (double)d * elem + 4.0 * B * H * (double)Nq;
}

double mha_fwd_flops(int B, int H, int N, int d, int causal) {
  const double f = 4.0 * B * H * (double)N * (double)N * d;
  return causal ? f / 2.0 : f;
}

double mha_fwd_bytes(int B, int H, int N, int d, mha_dtype dtype) {
  const double elem = dtype == MHA_DTYPE_F32 ? 4.0 : 2.0;
  return 4.0 * B * H * (double)N * d * elem + 4.0 * B * H * (double)N;
}

const char* mha_status_string(mha_status status) {
  switch (status) {
    case MHA_OK: return "MHA_OK: success";
    case MHA_ERR_INVALID_ARG: return "MHA_ERR_INVALID_ARG: invalid argument";
    case MHA_ERR_UNSUPPORTED: return "MHA_ERR_UNSUPPORTED: unsupported head dim, alignment or size";
    case MHA_ERR_HIP: return "MHA_ERR_HIP: the HIP runtime rejected the launch";
    case MHA_ERR_SCRATCH: return "MHA_ERR_SCRATCH: the call needs more than the library's static scratch";
  }
  return "unknown mha_status";
}

const char* mha_version(void) { return "mha-gfx950 0.1.0"; }

}  // extern "C"
