/*
 * mha.h -- C ABI of the fused multi-head attention forward library (libmha.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the FlashAttention-2 forward pass: Algorithm 1 ("FlashAttention-2
 * forward") of "ML-Triton, A Multi-Level Compilation and Language Extension to Triton
 * GPU Programming", section 2.5, which computes for every (batch b, head h) the
 * softmax-weighted sum of value rows defined in "Triton学习" (lorn3.bearblog.dev),
 * Puzzle 9 "Simple FlashAttention":
 *
 *     s_ij  = scale * <q_i, k_j>                      j visible to i
 *     O_i   = sum_j exp(s_ij - m_i) v_j / l_i,        m_i = max_j s_ij,
 *     l_i   = sum_j exp(s_ij - m_i),                  lse_i = m_i + ln(l_i)
 *
 * "visible" is every key, or with the causal mask only keys j <= i.
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, contiguous, row-major: Q, K, V, O are [B, H, N, d] (the last
 *     index fastest); LSE is [B, H, N] float32.  Query and key lengths are equal (N).
 *   - All tensor pointers are DEVICE pointers on the current HIP device, 16-byte
 *     aligned.  The caller owns every buffer; the library allocates nothing, keeps no
 *     state between calls and is safe to call from several threads.
 *   - O and LSE are fully overwritten.  Outputs must not overlap inputs.
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     default stream) and the function returns at once.  Completion is observed by
 *     synchronising that stream.
 *   - Errors are reported only through the return value.  Arguments are validated on
 *     the host before anything is enqueued; a rejected call touches no memory.
 */
#ifndef MHA_H_
#define MHA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mha_status {
  MHA_OK = 0,
  MHA_ERR_INVALID_ARG = 1, /* null pointer, B/H/N < 1, causal not 0/1, scale not finite,
                              unknown dtype */
  MHA_ERR_UNSUPPORTED = 2, /* head dim not 64 or 128, pointer not 16-byte aligned,
                              grid larger than the launch limit */
  MHA_ERR_HIP = 3          /* the HIP runtime rejected the launch */
} mha_status;

typedef enum mha_dtype {
  MHA_DTYPE_F32 = 0,  /* Q, K, V, O float32; all arithmetic in float32 */
  MHA_DTYPE_BF16 = 1, /* Q, K, V, O bfloat16; products accumulate in float32, the
                         softmax runs in float32, P is rounded to bfloat16 (round to
                         nearest even) before the second product, O is rounded once */
  MHA_DTYPE_F16 = 2   /* Q, K, V, O IEEE float16, as in the paged-attention listing
                         (ML-Triton paper, section 3.2, Figure 8, which casts P to
                         float16 before the second product); otherwise as bfloat16:
                         float32 accumulation and softmax, P and O rounded to float16
                         (round to nearest even) */
} mha_dtype;

/*
 * mha_fwd -- fused attention forward, Algorithm 1 of the ML-Triton paper (section 2.5).
 *
 *   q, k, v  device pointers to [B, H, N, d] tensors of `dtype` (read only)
 *   o        device pointer to the [B, H, N, d] output of `dtype`
 *   lse      device pointer to the [B, H, N] float32 output: per-row natural-log
 *            logsumexp of the scaled, masked logits (m_i + ln l_i above)
 *   B, H, N  batch, heads, sequence length (>= 1 each)
 *   d        head dimension: 64 or 128
 *   causal   0: every key visible; 1: key j visible to query i iff j <= i
 *   scale    multiplies q.k before the softmax (finite; usually 1/sqrt(d))
 *   dtype    element type of q, k, v, o
 *   stream   hipStream_t to enqueue on (NULL = default stream)
 *
 * Returns MHA_OK once the kernel is enqueued, else the error above.
 */
mha_status mha_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale,
                   mha_dtype dtype, void* stream);

/*
 * mha_fwd_validate -- the argument checks of mha_fwd alone, on the host, with no HIP
 * call.  Same arguments and same return value mha_fwd would give for a rejected call;
 * MHA_OK means mha_fwd would launch.
 */
mha_status mha_fwd_validate(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, int B, int H, int N, int d, int causal,
                            float scale, mha_dtype dtype);

/*
 * mha_fwd_flops -- the floating-point work credited to one mha_fwd call:
 * 4*B*H*N*N*d (two products of 2*N*N*d each per head), halved when causal.
 * Pure host function.
 */
double mha_fwd_flops(int B, int H, int N, int d, int causal);

/*
 * mha_fwd_bytes -- the algorithmic HBM traffic of one call: Q, K, V read once and O
 * written once (B*H*N*d elements each) plus the float32 LSE.  Pure host function.
 */
double mha_fwd_bytes(int B, int H, int N, int d, mha_dtype dtype);

/*
 * Split-KV forward (decoding with a long key/value sequence).
 *
 * The split-KV decomposition of the ML-Triton paper, section 3.2 (Flash Decoding splits
 * the keys and values of long KV sequences; Figure 10 partitions the KV cache and
 * reduces the partial results): Nq query rows (typically 1) per head attend to all Nk
 * keys of the head, with no mask.  The keys are cut into `splits` contiguous ranges;
 * every range yields a partial result (O_s normalised by its own row sum, and its
 * logsumexp lse_s), and the partials are merged exactly:
 *
 *     lse = log sum_s exp(lse_s),     O = sum_s exp(lse_s - lse) * O_s,
 *
 * which is the same O and lse as the definition above over all Nk keys.
 *
 *   q, o     [B, H, Nq, d] of `dtype`;  k, v  [B, H, Nk, d] of `dtype` (device pointers)
 *   lse      [B, H, Nq] float32
 *   splits   number of key ranges; 0 lets the library choose (mha_fwd_splitkv_splits)
 *   workspace, workspace_bytes
 *            caller-owned device memory of at least mha_fwd_splitkv_workspace_size(...)
 *            bytes, 16-byte aligned, holding the float32 partial results; its contents
 *            are scratch (overwritten, never read before written).  Calls that share a
 *            workspace must not overlap in time.
 *   other arguments as for mha_fwd.
 *
 * Errors as for mha_fwd, plus MHA_ERR_INVALID_ARG for Nq or Nk < 1, splits < 0, a null
 * workspace or one smaller than required.  Two kernels are enqueued on `stream`.
 */
mha_status mha_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, float scale, mha_dtype dtype,
                           int splits, void* workspace, size_t workspace_bytes, void* stream);

/* mha_fwd_splitkv_validate -- the argument checks of mha_fwd_splitkv alone, host only. */
mha_status mha_fwd_splitkv_validate(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, int B, int H, int Nq, int Nk, int d,
                                    float scale, mha_dtype dtype, int splits,
                                    const void* workspace, size_t workspace_bytes);

/*
 * mha_fwd_splitkv_splits -- the number of key ranges mha_fwd_splitkv will use for a
 * request of `splits` (0: automatic, about 512 workgroups with at least 512 keys per
 * range).  Every range is a whole number of 64-key tiles.  0 for invalid sizes.
 */
int mha_fwd_splitkv_splits(int B, int H, int Nq, int Nk, int splits);

/*
 * mha_fwd_splitkv_workspace_size -- bytes of workspace mha_fwd_splitkv needs:
 * resolved_splits * B * H * Nq * (d + 1) * 4.  0 for invalid sizes.  Host only.
 */
size_t mha_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d, int splits);

/*
 * mha_fwd_splitkv_bytes -- algorithmic HBM traffic of one mha_fwd_splitkv call: Q read
 * and O written (B*H*Nq*d elements each), K and V read once (B*H*Nk*d each), plus the
 * float32 LSE (the float32 partials are extra, implementation traffic).  Host only.
 */
double mha_fwd_splitkv_bytes(int B, int H, int Nq, int Nk, int d, mha_dtype dtype);

/* mha_status_string -- static, human-readable text for a status code. */
const char* mha_status_string(mha_status status);

/* mha_version -- static version string of the library build. */
const char* mha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H_ */
