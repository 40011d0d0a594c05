// Internal interface between the C ABI (mha_api.cpp) and the HIP kernels.
#ifndef MHA_LAUNCH_H_
#define MHA_LAUNCH_H_

#include <hip/hip_runtime_api.h>

namespace mha_impl {

// Query rows per workgroup of the forward kernel (the same for every element type).
int fwd_query_block(int dtype);

// Enqueue the forward kernel; arguments already validated.  dtype: 0 fp32, 1 bf16,
// 2 fp16 (the mha_dtype values).  Returns the launch status.
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int N, int d, int causal, float scale, int dtype, hipStream_t stream);

// Enqueue the split-KV forward (no mask; Nq query rows against Nk keys per head): the
// partial kernel over `splits` key ranges of `chunk` keys, then the merge.  part_o /
// part_lse: float32 [splits][B*H][Nq][d] and [splits][B*H][Nq].  Arguments validated.
hipError_t launch_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                              int Nq, int Nk, int d, float scale, int dtype, int splits, int chunk,
                              float* part_o, float* part_lse, hipStream_t stream);

// The static device scratch of the no-allocation split-KV entry point: its address on
// the current device (looked up once per device with hipGetSymbolAddress) and its size.
hipError_t scratch_address(void** out);
size_t scratch_bytes();

// Enqueue the paged split-KV forward: as launch_fwd_splitkv, with K and V gathered from
// block pools [num_blocks][H][2^bs_log2][d] through block_table [B][max_blocks]; sequence
// b uses keys [0, seq_lens[b]) (clamped to [0, max_blocks << bs_log2]).  part_o /
// part_lse are sized for `splits` ranges of `chunk` keys.  Arguments validated.
hipError_t launch_fwd_paged(const void* q, const void* k_pool, const void* v_pool, const int* block_table,
                            const int* seq_lens, void* o, float* lse, int B, int H, int Nq, int d, float scale,
                            int dtype, int num_blocks, int bs_log2, int max_blocks, int splits, int chunk,
                            float* part_o, float* part_lse, hipStream_t stream);

// Enqueue the dense GEMM C [M,N] = A [M,K] . B [K,N] (row-major, dtype 1 bf16 or 2 fp16,
// float32 accumulation, C in the input type).  Arguments validated.
hipError_t launch_gemm(const void* a, const void* b, void* c, int M, int N, int K, int dtype,
                       hipStream_t stream);

// Enqueue the split-K GEMM: `splits` ranges of `kchunk` keys of K (a multiple of 64),
// float32 partials in part [splits][M][N], then their sum rounded to C.  Validated.
hipError_t launch_gemm_splitk(const void* a, const void* b, void* c, int M, int N, int K, int dtype, int splits,
                              int kchunk, float* part, hipStream_t stream);

}  // namespace mha_impl

#endif  // MHA_LAUNCH_H_
