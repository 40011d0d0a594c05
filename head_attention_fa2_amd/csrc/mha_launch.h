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

}  // namespace mha_impl

#endif  // MHA_LAUNCH_H_
