// C ABI of libmha.so: argument validation on the host, then one kernel launch.
// The entry points and their contracts are declared in include/mha.h.
#include "mha.h"

#include <cmath>
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

}  // namespace

extern "C" {

mha_status mha_fwd_validate(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, int B, int H, int N, int d, int causal, float scale,
                            mha_dtype dtype) {
  return validate(q, k, v, o, lse, B, H, N, d, causal, scale, dtype);
}

mha_status mha_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, int causal, float scale, mha_dtype dtype, void* stream) {
  const mha_status st = validate(q, k, v, o, lse, B, H, N, d, causal, scale, dtype);
  if (st != MHA_OK) return st;
  const hipError_t e = mha_impl::launch_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, (int)dtype,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
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
  }
  return "unknown mha_status";
}

const char* mha_version(void) { return "mha-gfx950 0.1.0"; }

}  // extern "C"
