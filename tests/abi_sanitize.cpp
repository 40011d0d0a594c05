// Host-only driver of the C ABI layer (head_attention_fa2_amd/csrc/mha_api.cpp), built with
// g++ -fsanitize=address,undefined.  The HIP launchers are replaced by stubs that write, on
// the host, exactly the workspace region the kernels would write (partial O and partial
// LSE of every split), so an undersized workspace or a wrong partial-LSE offset becomes
// an AddressSanitizer report; UndefinedBehaviorSanitizer checks the size arithmetic of
// every *_validate, *_splits and *_workspace_size helper over extreme arguments.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "mha.h"
#include "mha_launch.h"

namespace {
int g_launches = 0;
int g_failures = 0;

void check(bool ok, const char* what, int line) {
  if (!ok) {
    std::printf("FAIL line %d: %s\n", line, what);
    ++g_failures;
  }
}
#define CHECK(x) check((x), #x, __LINE__)

// The split-KV kernels write partial O [splits][B*H][Nq][d] then partial LSE
// [splits][B*H][Nq] (float32); the stub writes both regions in full.
void touch_partials(float* part_o, float* part_lse, int B, int H, int Nq, int d, int splits) {
  const size_t rows = (size_t)splits * B * H * Nq;
  std::memset(part_o, 0, rows * d * sizeof(float));
  std::memset(part_lse, 0, rows * sizeof(float));
}
}  // namespace

namespace mha_impl {
int fwd_query_block(int) { return 128; }

// host stand-in for the static device scratch of mha_fwd_splitkv_noalloc: exactly its size
size_t scratch_bytes() { return MHA_SCRATCH_BYTES; }
hipError_t scratch_address(void** out) {
  static std::vector<char> host_scratch(MHA_SCRATCH_BYTES);
  *out = host_scratch.data();
  return hipSuccess;
}

hipError_t launch_fwd(const void*, const void*, const void*, void*, float*, int B, int H, int N, int d,
                      int causal, float scale, int dtype, hipStream_t) {
  ++g_launches;
  CHECK(B >= 1 && H >= 1 && N >= 1 && (d == 64 || d == 128) && (causal == 0 || causal == 1));
  CHECK(std::isfinite(scale) && dtype >= 0 && dtype <= 2);
  return hipSuccess;
}

hipError_t launch_fwd_splitkv(const void*, const void*, const void*, void*, float*, int B, int H, int Nq, int Nk,
                              int d, float, int, int splits, int chunk, float* part_o, float* part_lse,
                              hipStream_t) {
  ++g_launches;
  CHECK(splits >= 1 && chunk % 64 == 0 && (int64_t)splits * chunk >= Nk && (int64_t)(splits - 1) * chunk < Nk);
  touch_partials(part_o, part_lse, B, H, Nq, d, splits);
  return hipSuccess;
}

hipError_t launch_fwd_paged(const void*, const void*, const void*, const int*, const int*, void*, float*, int B,
                            int H, int Nq, int d, float, int, int num_blocks, int bs_log2, int max_blocks,
                            int splits, int chunk, float* part_o, float* part_lse, hipStream_t) {
  ++g_launches;
  const int64_t keys = (int64_t)max_blocks << bs_log2;
  CHECK(num_blocks >= 1 && bs_log2 >= 4 && bs_log2 <= 16);
  CHECK(splits >= 1 && chunk % 64 == 0 && (int64_t)splits * chunk >= keys && (int64_t)(splits - 1) * chunk < keys);
  touch_partials(part_o, part_lse, B, H, Nq, d, splits);
  return hipSuccess;
}

hipError_t launch_gemm(const void*, const void*, void*, int M, int N, int K, int dtype, hipStream_t) {
  ++g_launches;
  CHECK(M >= 1 && N % 8 == 0 && K % 8 == 0 && (dtype == 1 || dtype == 2));
  return hipSuccess;
}

hipError_t launch_gemm_splitk(const void*, const void*, void*, int M, int N, int K, int, int splits, int kchunk,
                              float* part, hipStream_t) {
  ++g_launches;
  CHECK(splits >= 1 && kchunk % 64 == 0 && (int64_t)splits * kchunk >= K && (int64_t)(splits - 1) * kchunk < K);
  std::memset(part, 0, (size_t)splits * M * N * sizeof(float));
  return hipSuccess;
}
}  // namespace mha_impl

int main() {
  alignas(16) static char buf[64];
  const void* p = buf;
  void* w = buf;
  float* lse = reinterpret_cast<float*>(buf);
  const float inf = std::numeric_limits<float>::infinity();
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const int big = std::numeric_limits<int>::max();
  const int ints[] = {-big - 1, -1, 0, 1, 2, 63, 64, 65, 127, 128, 129, 1000, 4096, 65536, 1 << 20, big};
  const int dims[] = {-1, 0, 1, 32, 64, 96, 128, 256, big};

  // ---- fused forward: validation over extreme sizes, then a launch for every accepted call
  for (int B : ints)
    for (int N : ints)
      for (int d : dims)
        for (int causal : {-1, 0, 1, 2})
          for (int dt : {-1, 0, 1, 2, 3}) {
            const mha_status v = mha_fwd_validate(p, p, p, p, lse, B, 3, N, d, causal, 0.5f, (mha_dtype)dt);
            const int before = g_launches;
            const mha_status r = mha_fwd(p, p, p, w, lse, B, 3, N, d, causal, 0.5f, (mha_dtype)dt, nullptr);
            CHECK(v == r);
            CHECK((g_launches - before) == (r == MHA_OK ? 1 : 0));
            (void)mha_fwd_flops(B, 3, N, d, causal);
            (void)mha_fwd_bytes(B, 3, N, d, (mha_dtype)dt);
          }
  for (float s : {inf, -inf, nan}) CHECK(mha_fwd_validate(p, p, p, p, lse, 1, 1, 8, 64, 0, s, MHA_DTYPE_BF16) ==
                                         MHA_ERR_INVALID_ARG);
  CHECK(mha_fwd_validate(buf + 4, p, p, p, lse, 1, 1, 8, 64, 0, 1.f, MHA_DTYPE_BF16) == MHA_ERR_UNSUPPORTED);
  CHECK(mha_fwd_validate(nullptr, p, p, p, lse, 1, 1, 8, 64, 0, 1.f, MHA_DTYPE_BF16) == MHA_ERR_INVALID_ARG);

  // ---- split-KV: the workspace is exactly the size the library asks for, allocated on the
  // host, and the launcher stub writes every byte the kernels would
  const int nqs[] = {1, 2, 4, 127, 128, 129, 300};
  const int nks[] = {1, 63, 64, 65, 511, 512, 513, 5000, 131072, 1 << 20};
  for (int B : {1, 2, 5})
    for (int Nq : nqs)
      for (int Nk : nks)
        for (int d : {64, 128})
          for (int splits : {0, 1, 2, 3, 7, 64, 5000}) {
            const int H = 3;
            const size_t ws = mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, splits);
            const int s = mha_fwd_splitkv_splits(B, H, Nq, Nk, splits);
            CHECK(ws > 0 && s >= 1);
            CHECK(ws == (size_t)s * B * H * Nq * (d + 1) * sizeof(float));
            if (ws > ((size_t)1 << 28)) continue;
            std::vector<float> space(ws / sizeof(float) + 4);
            float* aligned = space.data();
            while ((reinterpret_cast<uintptr_t>(aligned) & 15u) != 0) ++aligned;
            CHECK(mha_fwd_splitkv(p, p, p, w, lse, B, H, Nq, Nk, d, 0.125f, MHA_DTYPE_BF16, splits, aligned, ws,
                                  nullptr) == MHA_OK);
            CHECK(mha_fwd_splitkv_validate(p, p, p, p, lse, B, H, Nq, Nk, d, 0.125f, MHA_DTYPE_BF16, splits,
                                           aligned, ws - 1) == MHA_ERR_INVALID_ARG);
            (void)mha_fwd_splitkv_bytes(B, H, Nq, Nk, d, MHA_DTYPE_BF16);
          }
  // no-allocation form: the stub writes the partials into a host buffer of exactly
  // MHA_SCRATCH_BYTES, so accepting a call that needs more would be a heap overflow
  int noalloc_ok = 0, noalloc_rejected = 0;
  for (int B : {1, 4, 64, 1000})
    for (int Nq : {1, 16, 300})
      for (int Nk : {1, 4096, 131072, 1 << 22})
        for (int d : {64, 128})
          for (int splits : {0, 1, 64, 4096}) {
            const int H = 8;
            const size_t need = mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, splits);
            const mha_status r =
                mha_fwd_splitkv_noalloc(p, p, p, w, lse, B, H, Nq, Nk, d, 0.1f, MHA_DTYPE_BF16, splits, nullptr);
            CHECK(r == (need <= MHA_SCRATCH_BYTES ? MHA_OK : MHA_ERR_SCRATCH));
            (r == MHA_OK ? noalloc_ok : noalloc_rejected)++;
          }
  CHECK(noalloc_ok > 0 && noalloc_rejected > 0);
  CHECK(mha_fwd_splitkv_noalloc(nullptr, p, p, w, lse, 1, 1, 1, 8, 64, 1.f, MHA_DTYPE_BF16, 0, nullptr) ==
        MHA_ERR_INVALID_ARG);
  CHECK(mha_fwd_splitkv_noalloc(p, p, p, w, lse, 1, 1, 1, 8, 96, 1.f, MHA_DTYPE_BF16, 0, nullptr) ==
        MHA_ERR_UNSUPPORTED);

  for (int a : ints)
    for (int b : ints) {
      (void)mha_fwd_splitkv_splits(a, 2, b, a, b);
      (void)mha_fwd_splitkv_workspace_size(a, b, 2, b, 128, a);
      (void)mha_fwd_splitkv_validate(p, p, p, p, lse, a, 2, b, a, 64, 1.f, MHA_DTYPE_F16, 0, p, (size_t)-1);
    }

  // ---- paged
  alignas(16) static int32_t table[8];
  for (int bs : {-16, 0, 8, 16, 17, 32, 64, 256, 65536, 131072})
    for (int max_blocks : {-1, 0, 1, 2, 3, 100, 70000, big})
      for (int Nq : {1, 4, 129})
        for (int splits : {0, 1, 3}) {
          const int B = 2, H = 2, d = 128;
          const size_t ws = mha_fwd_paged_workspace_size(B, H, Nq, d, bs, max_blocks, splits);
          const int s = mha_fwd_paged_splits(B, H, Nq, bs, max_blocks, splits);
          CHECK((ws == 0) == (s == 0));
          if (ws == 0 || ws > ((size_t)1 << 28)) continue;
          std::vector<float> space(ws / sizeof(float) + 4);
          float* aligned = space.data();
          while ((reinterpret_cast<uintptr_t>(aligned) & 15u) != 0) ++aligned;
          CHECK(mha_fwd_paged(p, p, p, table, table, w, lse, B, H, Nq, d, 10, bs, max_blocks, 0.1f, MHA_DTYPE_F16,
                              splits, aligned, ws, nullptr) == MHA_OK);
          CHECK(mha_fwd_paged_validate(p, p, p, table, table, p, lse, B, H, Nq, d, 10, bs, max_blocks, 0.1f,
                                       MHA_DTYPE_F16, splits, aligned, ws - 1) == MHA_ERR_INVALID_ARG);
          CHECK(mha_fwd_paged_validate(p, p, p, reinterpret_cast<const int32_t*>(buf + 2), table, p, lse, B, H, Nq,
                                       d, 10, bs, max_blocks, 0.1f, MHA_DTYPE_F16, splits, aligned, ws) ==
                MHA_ERR_UNSUPPORTED);
          (void)mha_fwd_paged_bytes(B, H, Nq, (long long)max_blocks * bs, d, MHA_DTYPE_F16);
        }

  // ---- GEMM and split-K GEMM
  for (int M : ints)
    for (int N : {-8, 0, 8, 12, 64, 4096, 14336, big})
      for (int K : {-8, 0, 8, 200, 4096, 14336, big}) {
        const mha_status v = mha_gemm_validate(p, p, p, M, N, K, MHA_DTYPE_BF16);
        CHECK(mha_gemm(p, p, w, M, N, K, MHA_DTYPE_BF16, nullptr) == v);
        (void)mha_gemm_flops(M, N, K);
        (void)mha_gemm_bytes(M, N, K, MHA_DTYPE_BF16);
        (void)mha_gemm_splitk_splits(M, N, K, 0);
        (void)mha_gemm_splitk_workspace_size(M, N, K, 3);
      }
  for (int M : {1, 16, 100})
    for (int N : {8, 64, 4096})
      for (int K : {8, 64, 200, 4096, 14336})
        for (int splits : {0, 1, 2, 5, 1000}) {
          const size_t ws = mha_gemm_splitk_workspace_size(M, N, K, splits);
          CHECK(ws > 0);
          std::vector<float> space(ws / sizeof(float) + 4);
          float* aligned = space.data();
          while ((reinterpret_cast<uintptr_t>(aligned) & 15u) != 0) ++aligned;
          CHECK(mha_gemm_splitk(p, p, w, M, N, K, MHA_DTYPE_BF16, splits, aligned, ws, nullptr) == MHA_OK);
          CHECK(mha_gemm_splitk_validate(p, p, p, M, N, K, MHA_DTYPE_BF16, splits, aligned, ws - 1) ==
                MHA_ERR_INVALID_ARG);
        }

  for (int st = -1; st < 6; ++st) CHECK(mha_status_string((mha_status)st) != nullptr);
  CHECK(std::strlen(mha_version()) > 0);
  std::printf("launches %d, failures %d\n", g_launches, g_failures);
  if (g_failures == 0) std::printf("abi sanitize ok\n");
  return g_failures == 0 ? 0 : 1;
}
