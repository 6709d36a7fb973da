/*
 * dg.h - C ABI of the MI355X (gfx950) FP8 block-scaled NT GEMM library.
 *
 * What the library computes (D = A . B^T with fine-grained scales):
 *
 *   D[m, n] = bf16( sum over 128-wide K slabs kb of
 *                   (sum_{k in slab} A[m, k] * B[n, k]) * sfa[m, kb] * sfb[n / 128, kb] )
 *
 * A and B hold OCP e4m3 codes (1 byte, largest finite 448).  A carries one
 * fp32 scale per row and 128-wide K slab; B one fp32 scale per 128 x 128
 * block.  The operation and its MoE layouts are the ones described on the
 * DeepGEMM pages: "DeepSeek open-source week day 3" (deepseek.csdn.net),
 * section "technical features" (FP8 GEMM with fine-grained scaling and a
 * second, higher-precision accumulation level; contiguous and masked grouped
 * layouts); "DeepGEMM: making LLM matrix multiplication fly" (pomoai.com),
 * sections "core functions" (block-wise scaling) and "technical details"
 * (the fp8_gemm_nt naming: both operands K-contiguous).  The 1x128 / 128x128
 * granularity, e4m3 and the bf16 output are readings of those pages.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is caller-owned DEVICE memory (hipMalloc'd or a
 *   torch CUDA tensor) on the current device.  The library never frees,
 *   keeps or allocates anything on behalf of a call's arguments.
 * - Every compute call is asynchronous on `stream` (0 = the null stream),
 *   performs no host<->device copy and no synchronisation, and reads no
 *   device value on the host; every one can be captured into a HIP graph
 *   (see the workspace rule below).
 * - Split-K workspace.  Dense calls (fp8, bf16, fp4) whose K is split over
 *   several workgroups keep fp32 partial tiles and arrival counters in a
 *   library-owned workspace, one per (device, stream).  Calls on one stream
 *   share it in stream order; calls on different streams never share one, so
 *   split-K calls may overlap in time on different streams.  A call that
 *   needs more than its stream's workspace holds makes a larger one (one
 *   hipMalloc, then a zero-fill kernel on `stream`; the library frees
 *   nothing, so it adds no hipFree synchronisation); the smaller block is
 *   retired, not freed, and stays
 *   allocated until the process ends, because a launch in flight or a graph
 *   captured earlier may still use it.  While `stream` is capturing a graph
 *   such a growth is refused with DG_ERR_WORKSPACE and nothing is enqueued:
 *   size the workspace first with dg_reserve_workspace(bytes, stream), bytes
 *   from dg_dense_workspace_size.  A captured call keeps using the workspace
 *   its capture stream had; a replay must not overlap in time with other
 *   split-K work on that same workspace (replaying on the capture stream, or
 *   on any stream ordered with it, is safe).  dg_fp8_gemm_nt_noalloc uses a
 *   static per-GPU array instead and allocates nothing.
 * - Layouts are packed and row-major:
 *     A       [m][k]               (masked: [num_groups][max_m][k])
 *     B       [n][k]               (grouped: [num_groups][n][k])
 *     D       [m][n] bf16 bits     (masked: [num_groups][max_m][n])
 *     sfa     slab-major [k/128][ld], ld = dg_get_sfa_ld(m): sfa[kb*ld + row]
 *             (masked: [num_groups][k/128][dg_get_sfa_ld(max_m)])
 *     sfb     [ceil(n/128)][k/128] (grouped: [num_groups][ceil(n/128)][k/128])
 * - Preconditions checked on the host: non-null pointers, A/B/D/sfa/sfb
 *   16-byte aligned, k >= 128 and k % 128 == 0 (the bf16 and fp4 entry points
 *   state their own K rule), n >= 1, m >= 0.  m == 0 (or
 *   num_groups == 0 rows) is a successful no-op.  On a failed check nothing
 *   is enqueued, D is untouched and a status other than DG_OK is returned;
 *   dg_last_error_message() then describes the failure.
 * - D is overwritten (not accumulated) for valid rows only; every other
 *   element of D is left bit-for-bit untouched.
 * - No exception crosses this interface.  Every function may be called from
 *   several host threads at once (the workspace table is locked; the last
 *   error message is kept per thread).
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dg_stream_t; /* the same handle as hipStream_t */

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad count        */
  DG_ERR_UNSUPPORTED_SHAPE = 2, /* k not a multiple of 128, m not aligned, ...  */
  DG_ERR_MISALIGNED = 3,        /* a pointer not 16-byte aligned                 */
  DG_ERR_NO_DEVICE = 4,         /* no usable gfx950 device                       */
  DG_ERR_HIP = 5,               /* a HIP runtime call or kernel launch failed     */
  DG_ERR_INTERNAL = 6,
  DG_ERR_WORKSPACE = 7          /* the stream's split-K workspace would have to
                                   grow while the stream is capturing a graph */
} dg_status;

/*
 * Dense FP8 NT GEMM: D[m][n] = A[m][k] . B[n][k]^T with 1x128 (A) and
 * 128x128 (B) fp32 block scales.  Rows m and columns n may be any size >= 0
 * and >= 1 respectively; a partial last 128-row block of B uses its own scale
 * row of sfb.  When the output tiles alone cannot fill the GPU (skinny m,
 * or few tiles, as in one GPU's shard of a larger GEMM), the K dimension is
 * split over several workgroups whose fp32 partial tiles meet in the
 * stream's split-K workspace (see the conventions above) and are added in a
 * fixed order, so results stay bit-for-bit reproducible.  For m <= 16, on
 * shapes whose 128-wide K slabs of 64-row tiles fill one run of at least 12
 * slabs per CU, a kernel that deals those slabs to the workgroups in equal
 * runs is used instead; every other shape takes the tiled kernels.  The
 * choice never changes a result beyond the split-K summation order.
 */
int dg_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, dg_stream_t stream);

/*
 * dg_fp8_gemm_nt for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as dg_fp8_gemm_nt (bit for bit), but
 * a split-K call takes its fp32 partial tiles and arrival counters from a
 * static array of the library, one per GPU (16 MiB of partials and 16384
 * counters, held until the process ends), instead of the stream's workspace;
 * the call never allocates, frees or synchronises.  Each call clears the
 * counters it uses with a small kernel on `stream` before the GEMM.  A call
 * that would need more scratch than the array holds returns
 * DG_ERR_UNSUPPORTED_SHAPE with nothing enqueued (the 64 x 2112 x 7168
 * decode shape takes 3.6 MiB).  All calls on one GPU share the array, so
 * calls of this entry point that overlap in time on one GPU (two streams, or
 * two threads) race and give wrong results; dg_fp8_gemm_nt has no such
 * limit.
 */
int dg_fp8_gemm_nt_noalloc(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                           uint16_t* d, int m, int n, int k, dg_stream_t stream);

/*
 * MoE grouped GEMM, contiguous layout ("DeepSeek open-source week day 3",
 * technical features, MoE item on the contiguous layout): the rows of all
 * experts are stacked in A (m rows), experts share n and k, and
 * m_indices[r] (device int32, m entries) names the expert whose B row r
 * uses.  Each aligned block of dg_get_m_alignment_for_contiguous_layout()
 * rows must belong to one expert; rows tagged outside [0, num_groups)
 * (padding, conventionally -1) are neither computed nor written, nor are
 * rows whose tag differs from the expert of their block.
 * m must be a multiple of that alignment (else DG_ERR_UNSUPPORTED_SHAPE).
 */
int dg_m_grouped_fp8_gemm_nt_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                                        const float* sfb, uint16_t* d, const int32_t* m_indices,
                                        int m, int n, int k, int num_groups, dg_stream_t stream);

/*
 * MoE grouped GEMM, masked layout ("DeepSeek open-source week day 3",
 * technical features, MoE item on the masked layout; PPIO's evaluation,
 * masked-layout section, decode use): every expert g owns a fixed
 * max_m x k slab of A and max_m x n slab of D; masked_m[g] (device int32,
 * num_groups entries, clamped on the device to [0, max_m]) says how many
 * leading rows are valid.  Only valid rows are computed and written, so the
 * shapes never change and the call suits graph capture.  expected_m is a
 * host-side hint of the typical valid count per expert (0 = unknown); it
 * only steers the tile choice and never changes results (every tile gives
 * the same bits).  Counts up to 48 pick 128-row tiles, which stream B
 * fastest while every expert fits 128 rows but slow down when one does not
 * (max_m <= 128 picks them in any case); counts up to 80 a 256-row tile
 * with the same streaming schedule; larger or unknown counts the schedule
 * that overlaps the fullest experts' MFMA work with their loads.
 */
int dg_m_grouped_fp8_gemm_nt_masked(const uint8_t* a, const float* sfa, const uint8_t* b,
                                    const float* sfb, uint16_t* d, const int32_t* masked_m,
                                    int num_groups, int max_m, int n, int k, int expected_m,
                                    dg_stream_t stream);

/*
 * MoE FC1 + SwiGLU on the masked layout, with h requantised for the second
 * GEMM: the single-GPU slice of the fused MoE kernel the pages describe
 * (the popular-press article on DeepGEMM, yeyulingfeng.com, section 04 on
 * Mega MoE: dispatch, the first GEMM, the SwiGLU activation, the second GEMM
 * and combine in one kernel; dispatch and combine across GPUs are not part of
 * this call).
 * B holds each expert's FC1 weight as [gate; up]: rows 0..inter-1 are the
 * gate projection, rows inter..2*inter-1 the up projection.  For expert g
 * and valid row m (m < clamp(masked_m[g], 0, max_m)):
 *
 *   gate[j] = FP8 GEMM of A[g][m] with B[g][j]           (as dg_m_grouped_fp8_gemm_nt_masked,
 *   up[j]   = FP8 GEMM of A[g][m] with B[g][inter + j]    but kept in fp32)
 *   h[j]    = silu(gate[j]) * up[j],   silu(x) = x / (1 + exp(-x))
 *
 * and h is quantised with the activation rule of dg_quantize_a_1x128 (per
 * row and 128-wide block of h: amax floored at 1e-4, s = amax / 448,
 * code = e4m3(h / s)), all in fp32.  Layouts:
 *     A   [num_groups][max_m][k] e4m3, sfa [num_groups][k/128][dg_get_sfa_ld(max_m)]
 *     B   [num_groups][2*inter][k] e4m3, sfb [num_groups][2*inter/128][k/128]
 *     hq  [num_groups][max_m][inter] e4m3 codes (output)
 *     hs  [num_groups][inter/128][dg_get_sfa_ld(max_m)] fp32 scales (output)
 * hq and hs are exactly the A operand of a masked GEMM with k = inter, so
 * the second layer reads them without a conversion pass.  inter must be a
 * positive multiple of 128 and k of 128; pointers 16-byte aligned
 * (masked_m 4-byte).  Rows past an expert's count, and the padding entries
 * of hs, are left untouched.  expected_m is a hint as for the masked GEMM.
 * Errors as for the other entry points; nothing is allocated.
 */
int dg_m_grouped_fp8_gemm_nt_masked_swiglu(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                           uint8_t* hq, float* hs, const int32_t* masked_m, int num_groups,
                                           int max_m, int inter, int k, int expected_m, dg_stream_t stream);

/*
 * MoE FC1 + SwiGLU + FP8 requantisation on the contiguous layout: the
 * prefill side of dg_m_grouped_fp8_gemm_nt_masked_swiglu (the popular-press
 * article on DeepGEMM, yeyulingfeng.com, section on MoE: the contiguous
 * layout for prefill, the masked one for decode; section 04 on Mega MoE for
 * the fused FC1 and SwiGLU).  B holds each expert's FC1 weight as [gate; up]
 * as for the masked entry point, and for every row m whose tag
 * e = m_indices[m] lies in [0, num_groups):
 *
 *   gate[j] = FP8 GEMM of A[m] with B[e][j]           (as dg_m_grouped_fp8_gemm_nt_contiguous,
 *   up[j]   = FP8 GEMM of A[m] with B[e][inter + j]    but kept in fp32)
 *   h[j]    = silu(gate[j]) * up[j]
 *
 * quantised with the activation rule of dg_quantize_a_1x128, all in fp32.
 * Layouts:
 *     A   [m][k] e4m3, sfa [k/128][dg_get_sfa_ld(m)], m_indices [m] (-1 = padding)
 *     B   [num_groups][2*inter][k] e4m3, sfb [num_groups][2*inter/128][k/128]
 *     hq  [m][inter] e4m3 codes (output)
 *     hs  [inter/128][dg_get_sfa_ld(m)] fp32 scales (output)
 * hq and hs are exactly the A operand of a contiguous GEMM with k = inter
 * and the same m_indices.  m must be a multiple of the 128-row alignment
 * (every 128-row block holds one expert's rows and padding); inter a
 * positive multiple of 128, k of 128; pointers 16-byte aligned (m_indices
 * 4-byte).  Padding rows, rows with an out-of-range tag and the padding
 * entries of hs are left untouched.  Errors as for the other entry points;
 * nothing is allocated.
 */
int dg_m_grouped_fp8_gemm_nt_contiguous_swiglu(const uint8_t* a, const float* sfa, const uint8_t* b,
                                               const float* sfb, uint8_t* hq, float* hs, const int32_t* m_indices,
                                               int m, int inter, int k, int num_groups, dg_stream_t stream);

/*
 * BF16 NT GEMM: D[m][n] = bf16( sum_k A[m, k] * B[n, k] ) for bf16 A [m][k]
 * and B [n][k] (bit patterns in uint16), fp32 accumulation, no scales
 * ("DeepGEMM: making LLM matrix multiplication fly", pomoai.com, core
 * functions: BF16 GEMMs beside the FP8 ones).  The same tiles, LDS layout and
 * split-K as the FP8 dense GEMM run it on gfx950's bf16 MFMA
 * (v_mfma_f32_16x16x32_bf16).  k must be a positive multiple of 64 (one
 * 128-byte slab row); otherwise as dg_fp8_gemm_nt (m may be 0, n >= 1,
 * 16-byte aligned pointers, the split-K workspace note applies).
 */
int dg_bf16_gemm_nt(const uint16_t* a, const uint16_t* b, uint16_t* d, int m, int n, int k, dg_stream_t stream);

/*
 * FP4 NT GEMM ("DeepGEMM: making LLM matrix multiplication fly", pomoai.com,
 * core functions: FP4 named beside FP8 and BF16; its caveats warn that FP4
 * may cost accuracy).  The pages give FP4 no scaling rule, so the FP8 method
 * carries over with e2m1 operands:
 *
 *   D[m][n] = bf16( sum over slabs kb of
 *                   (sum_{k in kb} A[m, k] * B[n, k]) * sfa[m, kb] * sfb[n / 128, kb] )
 *
 * A [m][k/2] and B [n][k/2] hold e2m1 codes two per byte (element 2i in the
 * low nibble of byte i); sfa (slab-major, dg_get_sfa_ld(m)) and sfb
 * ([ceil(n/128)][k/128]) are the FP8 scale layouts.  k must be a positive
 * multiple of 256 (whole 128-byte rows); otherwise as dg_fp8_gemm_nt (m may
 * be 0, n >= 1, 16-byte aligned pointers, the split-K workspace note).
 */
int dg_fp4_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d,
                   int m, int n, int k, dg_stream_t stream);

/*
 * K-grouped GEMM ("DeepGEMM: making LLM matrix multiplication fly",
 * pomoai.com, core functions: the K-grouped family beside the M-grouped one,
 * for the irregular shapes of MoE training such as weight gradients, where
 * the tokens of each expert form a run of K).  The groups are concatenated
 * along K: group g owns the k_sizes[g] K columns that follow the groups
 * before it, and
 *
 *   D[g][m][n] = bf16( sum over group g's slabs kb of
 *                      (sum_{k in slab kb} A[m, k] * B[n, k]) * sfa[m, kb] * sfb[n / 128, kb] )
 *
 * with the dense layouts and scales for A [m][k], sfa (slab-major,
 * dg_get_sfa_ld(m)), B [n][k] and sfb [ceil(n/128)][k/128]; D is
 * [num_groups][m][n] bf16.  k_sizes is device int32 (num_groups entries),
 * read only on the device so that the call is graph-capturable: each size
 * must be a multiple of 128 and their sum at most k; on the device a
 * negative size counts as 0, the remainder below a multiple of 128 is
 * ignored, and a group is cut off at k.  A group with no K columns gets
 * D[g] = 0.  Every element of D is written.
 */
int dg_k_grouped_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                             uint16_t* d, const int32_t* k_sizes, int num_groups, int m, int n, int k,
                             dg_stream_t stream);

/* Row alignment required of each expert's segment in the contiguous layout (128). */
int dg_get_m_alignment_for_contiguous_layout(void);

/* Leading dimension of the slab-major sfa layout for m rows: m rounded up to 4. */
int dg_get_sfa_ld(int m);

/*
 * Quantise an fp32 activation matrix x[m][k] to e4m3 codes q[m][k] with one
 * fp32 scale per row and 128-wide slab, written slab-major to
 * sfa[kb*dg_get_sfa_ld(m) + row] (entries for rows >= m are set to 0).
 * Per block: amax = max|x| (floored at 1e-4), s = amax / 448 (fp32, correctly
 * rounded), q = e4m3(x / s) rounded to nearest even and saturated at 448.
 */
int dg_quantize_a_1x128(const float* x, uint8_t* q, float* sfa, int m, int k, dg_stream_t stream);

/*
 * Quantise an fp32 weight matrix x[n][k] to e4m3 codes q[n][k] with one fp32
 * scale per 128 x 128 block, sfb[ceil(n/128)][k/128]; same rule as above;
 * the last row block may be partial.
 */
int dg_quantize_b_128x128(const float* x, uint8_t* q, float* sfb, int n, int k, dg_stream_t stream);

/*
 * FP4 quantisers: as dg_quantize_a_1x128 / dg_quantize_b_128x128 with e2m1
 * codes (range 6): per block amax (floored at 1e-4), s = amax / 6 (fp32,
 * correctly rounded), code = e2m1(x / s) rounded to nearest with ties to
 * even, saturated at 6.  q is [m][k/2] (resp. [n][k/2]) bytes, two codes per
 * byte, element 2i in the low nibble; the scale layouts are the FP8 ones.
 */
int dg_quantize_a_1x128_fp4(const float* x, uint8_t* q, float* sfa, int m, int k, dg_stream_t stream);
int dg_quantize_b_128x128_fp4(const float* x, uint8_t* q, float* sfb, int n, int k, dg_stream_t stream);

/*
 * Size the split-K workspace of `stream` on the current device to hold at
 * least `bytes` of partial tiles (dg_dense_workspace_size gives a call's
 * need), so that later calls on that stream that fit allocate nothing and
 * can be captured.  Growing allocates one block and enqueues a zero-fill
 * kernel on `stream`; it does not synchronise the device.  Returns
 * DG_ERR_WORKSPACE, with nothing done, if it would have to grow while
 * `stream` is capturing.
 */
int dg_reserve_workspace(size_t bytes, dg_stream_t stream);

/* Operand types of the dense entry points, for dg_dense_workspace_size. */
typedef enum { DG_DTYPE_FP8 = 0, DG_DTYPE_BF16 = 1, DG_DTYPE_FP4 = 2 } dg_dtype;

/*
 * Bytes of split-K workspace that a dense call of this dtype and shape
 * (dg_fp8_gemm_nt, dg_bf16_gemm_nt or dg_fp4_gemm_nt, m x n, K of k values)
 * needs on the current device: 0 when the call does not split K.  Passing
 * it to dg_reserve_workspace for a stream before capturing such calls on
 * that stream keeps them from allocating.  Same shape checks as the GEMM calls (k a positive
 * multiple of 128, 64 or 256 for fp8, bf16 and fp4, m >= 0, n >= 1), an
 * unknown dtype is DG_ERR_INVALID_ARGUMENT, and *bytes is 0 on any error.
 */
int dg_dense_workspace_size(int dtype, int m, int n, int k, size_t* bytes);

/* Static text for a status code. */
const char* dg_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* dg_last_error_message(void);

/*
 * Profiling hook: the next GEMM launch made on the calling thread records
 * `start_event` and `stop_event` (hipEvent_t handles created by the caller
 * with timing enabled; either may be NULL) at the start and end of the
 * kernel itself (hipExtLaunchKernel), so hipEventElapsedTime gives the
 * kernel's own duration without launch gaps.  One-shot: the hook clears
 * itself after that launch.  Not graph-capturable; for measurement only.
 */
int dg_profile_next_launch(void* start_event, void* stop_event);

/* Library version string. */
const char* dg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
