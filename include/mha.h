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
#include <stdint.h>

/* hipStream_t as the HIP runtime defines it (a pointer to the opaque ihipStream_t), so
 * that this header needs no HIP include: a caller that includes hip_runtime_api.h gets
 * the same type, and any caller may pass NULL or a stream handle from another binding
 * (for instance torch.cuda.current_stream().cuda_stream). */
#if !defined(HIP_INCLUDE_HIP_HIP_RUNTIME_API_H)
typedef struct ihipStream_t* hipStream_t;
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mha_status {
  MHA_OK = 0,
  MHA_ERR_INVALID_ARG = 1, /* null pointer, B/H/N < 1, causal not 0/1, scale not finite,
                              unknown dtype */
  MHA_ERR_UNSUPPORTED = 2, /* head dim not 64 or 128, pointer not 16-byte aligned,
                              grid larger than the launch limit */
  MHA_ERR_HIP = 3,         /* the HIP runtime rejected the launch */
  MHA_ERR_SCRATCH = 4      /* mha_fwd_splitkv_noalloc: the call needs more than the
                              library's static scratch (MHA_SCRATCH_BYTES) */
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
                   mha_dtype dtype, hipStream_t stream);

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
 * workspace or one smaller than required.  The partial kernel and, with more than one
 * range, the merge kernel are enqueued on `stream`; with a single range the partial
 * kernel writes O and lse itself and the workspace is not written.
 */
mha_status mha_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, float scale, mha_dtype dtype,
                           int splits, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mha_fwd_splitkv_noalloc -- mha_fwd_splitkv for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the float32 partial results go to a static device buffer of the library
 * (MHA_SCRATCH_BYTES bytes on every GPU it runs on, held until the process ends) instead
 * of a caller workspace.  The call allocates nothing; the caller passes q, k, v, o and
 * lse as for mha_fwd_splitkv, and the results are those of mha_fwd_splitkv with the same
 * arguments.
 *
 * The buffer's address on the current device is looked up on the first call made with
 * that device current.  Every call on one GPU shares that GPU's buffer: calls that
 * overlap in time on one GPU (different streams, host threads) race and must be ordered
 * by the caller.  Nothing in the buffer needs clearing: each call writes every partial
 * it reads.
 *
 * Errors as for mha_fwd_splitkv (without the workspace checks), plus MHA_ERR_SCRATCH when
 * mha_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, splits) exceeds MHA_SCRATCH_BYTES, and
 * MHA_ERR_HIP if the buffer's address cannot be obtained.
 */
#define MHA_SCRATCH_BYTES ((size_t)16 << 20)
mha_status mha_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int B, int H, int Nq, int Nk, int d, float scale, mha_dtype dtype,
                                   int splits, hipStream_t stream);

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

/*
 * Paged split-KV forward (decoding against a paged key/value cache).
 *
 * The paged attention of the ML-Triton paper, section 3.2 (Figures 8 and 9) and
 * section 4.3: each sequence's keys and values sit in fixed-size blocks scattered over
 * a pool and are reached through a block table; the attention is unchanged.  The
 * pages fix no layout, so this library defines one:
 *
 *   k_pool, v_pool  [num_blocks, H, block_size, d] of `dtype` (device): a block holds
 *                   block_size consecutive keys of every head, each head's rows
 *                   contiguous;
 *   block_table     [B, max_blocks] int32 (device): key j of sequence b is row
 *                   j % block_size of physical block block_table[b][j / block_size];
 *   seq_lens        [B] int32 (device): sequence b has keys 0 .. seq_lens[b]-1;
 *   q, o            [B, H, Nq, d] of `dtype`;  lse  [B, H, Nq] float32 (device).
 *
 * Every query row of sequence b attends to all of its keys (no mask); O and lse are
 * those of the definition above over the gathered keys, computed with the split-KV
 * merge.  A sequence with no keys gives O = 0 and lse = -inf.  The table and the
 * lengths are read on the device only: a length is clamped to [0, max_blocks *
 * block_size] and a table entry into [0, num_blocks), so bad values give wrong
 * numbers, never an access outside the pools; entries past a sequence's last block
 * are never used.
 *
 *   block_size  a power of two, 16 .. 65536 (else MHA_ERR_UNSUPPORTED)
 *   splits      key ranges per sequence over max_blocks * block_size keys; 0 =
 *               automatic (mha_fwd_paged_splits).  A range past a sequence's end
 *               costs one workgroup that exits at once.  With a single range no merge
 *               is launched (as for mha_fwd_splitkv).
 *   workspace   as for mha_fwd_splitkv, of at least mha_fwd_paged_workspace_size(...)
 *               bytes.
 *   other arguments as for mha_fwd_splitkv.
 *
 * Errors as for mha_fwd_splitkv, with MHA_ERR_INVALID_ARG for a null table, lengths
 * or pool, num_blocks or max_blocks < 1, and MHA_ERR_UNSUPPORTED for a table or
 * lengths pointer not 4-byte aligned or max_blocks * block_size above 2^30.
 */
mha_status mha_fwd_paged(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                         int B, int H, int Nq, int d, int num_blocks, int block_size,
                         int max_blocks, float scale, mha_dtype dtype, int splits,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mha_fwd_paged_splits -- the number of key ranges mha_fwd_paged will use for a request
 * of `splits` (0: automatic, as mha_fwd_splitkv_splits with Nk = max_blocks *
 * block_size).  0 for invalid sizes.  Host only.
 */
int mha_fwd_paged_splits(int B, int H, int Nq, int block_size, int max_blocks, int splits);

/*
 * mha_fwd_paged_workspace_size -- bytes of workspace mha_fwd_paged needs:
 * resolved_splits * B * H * Nq * (d + 1) * 4.  0 for invalid sizes.  Host only.
 */
size_t mha_fwd_paged_workspace_size(int B, int H, int Nq, int d, int block_size, int max_blocks,
                                    int splits);

/* mha_fwd_paged_validate -- the argument checks of mha_fwd_paged alone, host only. */
mha_status mha_fwd_paged_validate(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  const void* o, const float* lse, int B, int H, int Nq, int d,
                                  int num_blocks, int block_size, int max_blocks, float scale,
                                  mha_dtype dtype, int splits, const void* workspace,
                                  size_t workspace_bytes);

/*
 * mha_fwd_paged_bytes -- algorithmic HBM traffic of one mha_fwd_paged call over
 * total_keys keys in all (the sum of seq_lens): Q read and O written, the K and V rows
 * of every key read once, plus the float32 LSE.  Table and length reads (4 bytes per
 * block and per sequence) and the float32 partials are not counted.  Host only.
 */
double mha_fwd_paged_bytes(int B, int H, int Nq, long long total_keys, int d, mha_dtype dtype);

/*
 * Dense GEMM.
 *
 * The tiled contraction of the ML-Triton paper, section 2 (a workgroup accumulates its
 * block of C over k-steps in float32 and stores it once) and section 4.1 (compute-bound
 * GEMMs from LLM layers):
 *
 *     C[m][n] = sum_k A[m][k] * B[k][n]
 *
 *   a       [M, K] row-major, b [K, N] row-major, c [M, N] row-major (device pointers),
 *           all of `dtype`: MHA_DTYPE_BF16 or MHA_DTYPE_F16.  Products are accumulated
 *           in float32 and C is rounded once to `dtype` (round to nearest even).  C
 *           must not overlap A or B.
 *   M, N, K >= 1; N and K multiples of 8 (16-byte rows); A and B under 4 GiB each.
 *   stream  hipStream_t (NULL = default stream); one kernel is enqueued.
 *
 * Errors: MHA_ERR_INVALID_ARG for a null pointer, a size < 1 or an unknown dtype;
 * MHA_ERR_UNSUPPORTED for fp32, N or K not a multiple of 8, a pointer not 16-byte
 * aligned, an operand of 4 GiB or more, or more than 2^31 - 1 blocks of 128 x 64;
 * MHA_ERR_HIP if the launch fails.
 */
mha_status mha_gemm(const void* a, const void* b, void* c, int M, int N, int K, mha_dtype dtype,
                    hipStream_t stream);

/* mha_gemm_validate -- the argument checks of mha_gemm alone, host only. */
mha_status mha_gemm_validate(const void* a, const void* b, const void* c, int M, int N, int K,
                             mha_dtype dtype);

/*
 * Split-K GEMM, for the memory-bound shapes of the ML-Triton paper's section 4.1 (one
 * small dimension, as in next-token prediction, where the tiles of C alone cannot
 * occupy the GPU).  The same C = A.B as mha_gemm (same arguments and errors); K is cut
 * into `splits` ranges, each workgroup accumulates one range of one 128 x 128 block of C
 * in float32, and a second kernel adds the float32 partials and rounds the sum once to
 * `dtype`.  The result is within the same bound as mha_gemm's (a float32-accumulated,
 * once-rounded sum), summed in a different order.
 *
 *   splits      K ranges; 0 = automatic (mha_gemm_splitk_splits: the largest power of
 *               two within about 512 workgroups and at least 4 steps of 64 per range;
 *               the ranges are whole steps, so fewer may remain non-empty).
 *   workspace, workspace_bytes
 *               caller-owned device memory of at least mha_gemm_splitk_workspace_size(...)
 *               bytes, 16-byte aligned, for the partials [splits][M][N] float32 (scratch;
 *               calls that share it must not overlap in time).
 *
 * Errors as for mha_gemm, plus MHA_ERR_INVALID_ARG for splits < 0 or a null or too small
 * workspace, MHA_ERR_UNSUPPORTED for a workspace not 16-byte aligned or M*N >= 2^31.
 * Two kernels are enqueued on `stream`.
 */
mha_status mha_gemm_splitk(const void* a, const void* b, void* c, int M, int N, int K, mha_dtype dtype,
                           int splits, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* mha_gemm_splitk_validate -- the argument checks of mha_gemm_splitk alone, host only. */
mha_status mha_gemm_splitk_validate(const void* a, const void* b, const void* c, int M, int N, int K,
                                    mha_dtype dtype, int splits, const void* workspace,
                                    size_t workspace_bytes);

/* mha_gemm_splitk_splits -- K ranges mha_gemm_splitk uses for a request; 0 if invalid. */
int mha_gemm_splitk_splits(int M, int N, int K, int splits);

/* mha_gemm_splitk_workspace_size -- resolved_splits * M * N * 4 bytes; 0 if invalid. */
size_t mha_gemm_splitk_workspace_size(int M, int N, int K, int splits);

/* mha_gemm_flops -- 2*M*N*K, the credited work of one mha_gemm call.  Host only. */
double mha_gemm_flops(int M, int N, int K);

/*
 * mha_gemm_bytes -- algorithmic HBM traffic of one mha_gemm call: A and B read once,
 * C written once.  Host only.
 */
double mha_gemm_bytes(int M, int N, int K, mha_dtype dtype);

/* mha_status_string -- static, human-readable text for a status code. */
const char* mha_status_string(mha_status status);

/* mha_version -- static version string of the library build. */
const char* mha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H_ */
