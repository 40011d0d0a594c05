// Internal interface between the C ABI (mha_api.cpp) and the HIP kernels.
#ifndef MHA_LAUNCH_H_
#define MHA_LAUNCH_H_

#include <hip/hip_runtime_api.h>

namespace mha_impl {

// Query rows per workgroup of the forward kernel for bf16 (is_bf16 = 1) or fp32 inputs.
int fwd_query_block(int is_bf16);

// Enqueue the forward kernel; arguments already validated.  Returns the launch status.
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                      int N, int d, int causal, float scale, int is_bf16, hipStream_t stream);

}  // namespace mha_impl

#endif  // MHA_LAUNCH_H_
