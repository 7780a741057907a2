/*
 * tri_attn.h — C ABI of the gfx950 (MI355X) triangle-attention library, libtriattn.so.
 *
 * The operation is starting-node triangular attention as used in AlphaFold3-style
 * models ("TurboPairFormer: Fast and Stable Protein Folding Model Training with an
 * Optimized Triangle Attention Kernel", arXiv 2610.05854, Abstract).  For every batch
 * b, slice i and head h, with alpha = 1/sqrt(D):
 *
 *   s[j,k] = alpha * sum_c q[b,i,h,j,c] k[b,i,h,k,c] + bias[b,h,j,k] + m[b,i,k]
 *   o[b,i,h,j,:] = sum_k softmax_k(s[j,:]) v[b,i,h,k,:]
 *
 * where the pair bias is shared by all N slices and m = -inf for a masked key, else 0 (a
 * masked key is left out of the softmax; an additive -1e9 gives the same result for every
 * row that keeps a key).  The backward returns dq, dk, dv and dbias[b,h,j,k] =
 * sum_i dS[b,i,h,j,k], the reduction across slices that the shared bias adds (same Abstract).
 *
 * Rows with no key of finite score -- every key of the slice masked (a padded residue of a
 * cropped batch), or every key of the query carrying a -inf bias -- attend to nothing: their
 * output and residual are 0, their lse is +inf, and they contribute nothing to any gradient.
 *
 * Bias values are finite or -inf (a -inf bias removes that key for that query).  Finite bias
 * values are clamped to [-65504, 65504] in both passes (the backward streams the bias as
 * fp16); below that magnitude the bias is used exactly.  A bias of +inf is not supported.
 *
 * Memory layouts (row-major, contiguous, caller-owned DEVICE memory):
 *   q, k, v, o, residual, dO, dq, dk, dv : bf16 [B, N, H, N, D]   index [b, i, h, j, c]
 *   bias                                 : bf16 [B, H, N, N]      index [b, h, j, k]
 *   key_mask (optional)                  : uint8 [B, N, N]        index [b, i, k]; 1 keep, 0 mask
 *   lse                                  : fp32 [B, N, H, N]      natural-log logsumexp of each row
 *   dbias                                : fp32 [B, H, N, N]
 *
 * Conventions shared by every entry point:
 *   - All pointers are device pointers, 16-byte aligned (key_mask: any alignment).
 *   - Supported shapes: D in {16, 32}; B, H >= 1; 1 <= N <= TRI_ATTN_MAX_N for the backward
 *     (and the forward that feeds it), 1 <= N <= TRI_ATTN_FWD_MAX_N for the forward alone.
 *   - The library allocates no memory and keeps no state between calls (the one exception,
 *     tri_attn_fwd_noalloc below, keeps a fixed scratch array per GPU).  Scratch space comes
 *     from the caller through (workspace, workspace_bytes), sized by the matching
 *     *_workspace_bytes function, and is only valid for the call it is passed to.
 *   - Arguments are validated synchronously before anything is launched.  On any
 *     error nothing is launched and no output is written.
 *   - Work is enqueued on `stream` and runs asynchronously; faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - Outputs are overwritten, never accumulated into; outputs must not overlap inputs.
 *   - Every floating-point reduction runs in a fixed order that depends only on the
 *     shape, with no floating-point atomics: repeated calls with the same inputs and
 *     shape on the same device return bitwise-identical outputs.
 *   - Inputs (q, k, v, dO) are finite, and every score alpha*q.k + bias of a kept key stays
 *     within +-2^99 (the kernels mark masked keys with -2^100 internally).
 */
#ifndef TRI_ATTN_H
#define TRI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest N of the backward (and of a forward that feeds it).  Up to N = 768 a work-group keeps
 * the pair-bias gradient of all queries of its 64-key block in registers; longer slices are
 * split into ceil(N / 768) query chunks of near-equal size, whose dK / dV are summed in FP32
 * in chunk order (the workspace grows by 2 * chunks * B*N*H*N*D * 4 bytes). */
#define TRI_ATTN_MAX_N 2048
/* Largest N of the forward alone (inference on longer crops): the forward streams keys and has
 * no such per-query state. */
#define TRI_ATTN_FWD_MAX_N 4096

typedef enum {
  TRI_ATTN_SUCCESS = 0,
  TRI_ATTN_ERROR_INVALID_VALUE = 1, /* NULL required pointer, B/N/H < 1, output overlapping an input,
                                       unknown stage bits or layout */
  TRI_ATTN_ERROR_UNSUPPORTED = 2,   /* D not in {16, 32}, N above the call's limit, B > 2^20, H > 4096,
                                       B*N*H*ceil(N/128)*8 > 2^31 - 1, or a layout whose slice
                                       span exceeds 32-bit offsets */
  TRI_ATTN_ERROR_MISALIGNED = 3,    /* a tensor pointer that is not 16-byte aligned */
  TRI_ATTN_ERROR_WORKSPACE = 4,     /* workspace NULL or smaller than *_workspace_bytes() */
  TRI_ATTN_ERROR_LAUNCH = 5,        /* the HIP runtime rejected a kernel launch */
  TRI_ATTN_ERROR_SCRATCH_LIMIT = 6  /* tri_attn_fwd_noalloc: the shape needs more than
                                       TRI_ATTN_NOALLOC_SCRATCH_BYTES of scratch */
} tri_attn_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *tri_attn_status_string(int status);

/* Bytes of device workspace tri_attn_fwd needs for this shape (0 if the shape is invalid). */
size_t tri_attn_fwd_workspace_bytes(int64_t B, int64_t N, int64_t H, int64_t D);

/*
 * Forward: writes o, lse and (optionally) the output-rounding residual.
 *
 * residual: if non-NULL, receives bf16(o_fp32 - float(o)), the rounding error of the
 *   bf16 output kept at bf16 precision ("output-residual compensation", TurboPairFormer
 *   Abstract).  The bf16 output o itself does not depend on whether residual is stored.
 *   Pass NULL to skip it.
 * key_mask: NULL means no mask.
 */
tri_attn_status tri_attn_fwd(int64_t B, int64_t N, int64_t H, int64_t D,
                             const void *q, const void *k, const void *v, const void *bias,
                             const uint8_t *key_mask,
                             void *o, float *lse, void *residual,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace tri_attn_bwd needs for this shape (0 if the shape is invalid). */
size_t tri_attn_bwd_workspace_bytes(int64_t B, int64_t N, int64_t H, int64_t D);

/*
 * Backward: given the forward's o, lse (and residual) and the output gradient dO,
 * writes dq, dk, dv (bf16) and dbias (fp32).
 *
 * The softmax backward correction D[j] = sum_c dO[j,c] * o_fp32[j,c] is computed in
 * FP32 from o + residual when residual is non-NULL (compensated), or from the bf16 o
 * alone when residual is NULL.  dv does not depend on this choice.
 *
 * A key-tile-parallel kernel recomputes each probability tile once for dk, dv and dbias and
 * sums dbias over slices on chip, then over slice groups through ordered partial buffers held
 * in the workspace (TurboPairFormer Abstract: probability recomputation, ordered partial
 * reductions, no stored score gradient).  dq sums over every key: a query-tile kernel
 * recomputes the probability and score-gradient tiles once more and sums dq in FP32 in key
 * order, rounding once.  Every sum runs in a fixed order, so results are bitwise reproducible.
 */
tri_attn_status tri_attn_bwd(int64_t B, int64_t N, int64_t H, int64_t D,
                             const void *q, const void *k, const void *v, const void *bias,
                             const uint8_t *key_mask,
                             const void *o, const float *lse, const void *residual,
                             const void *dO,
                             void *dq, void *dk, void *dv, float *dbias,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Staged forms of the two calls, for callers that interleave their own work or time the
 * kernels individually.  tri_attn_fwd / tri_attn_bwd are exactly the staged call with
 * TRI_ATTN_STAGE_ALL.  Stages must run in ascending order, on one stream, with the same
 * arguments and the same workspace; the workspace carries intermediate results from one
 * stage to the next.  Validation is the same as for the unstaged call.
 *   forward : PREP = bias conversion into the workspace; MAIN = attention kernel; FINAL = none
 *   backward: PREP = bias conversion and the query-tile kernel (dq, and the correction D for
 *             the next stage); MAIN = the key-tile-parallel kernel (dk, dv, dbias partials);
 *             FINAL = the ordered sum of the dbias partials
 */
#define TRI_ATTN_STAGE_PREP 1u
#define TRI_ATTN_STAGE_MAIN 2u
#define TRI_ATTN_STAGE_FINAL 4u
#define TRI_ATTN_STAGE_ALL 7u

tri_attn_status tri_attn_fwd_stages(unsigned stages, int64_t B, int64_t N, int64_t H, int64_t D,
                                    const void *q, const void *k, const void *v, const void *bias,
                                    const uint8_t *key_mask,
                                    void *o, float *lse, void *residual,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

tri_attn_status tri_attn_bwd_stages(unsigned stages, int64_t B, int64_t N, int64_t H, int64_t D,
                                    const void *q, const void *k, const void *v, const void *bias,
                                    const uint8_t *key_mask,
                                    const void *o, const float *lse, const void *residual,
                                    const void *dO,
                                    void *dq, void *dk, void *dv, float *dbias,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Token-tensor layouts: where entry (b, slice i, head h, token j, channel c) of q, k, v, o,
 * residual, dO, dq, dk and dv lives.  All nine tensors of a call share one layout; each is
 * still one dense, 16-byte aligned block of B*N*N*H*D bf16 values.
 *
 *   TRI_ATTN_LAYOUT_SLICE_HEAD  [B, N, H, N, D], index [b, i, h, j, c] (the layout above)
 *   TRI_ATTN_LAYOUT_PAIR_START  [B, N, N, H, D], index [b, i, j, h, c]: the pair layout, heads
 *                               innermost, attending along the second pair index (starting node)
 *   TRI_ATTN_LAYOUT_PAIR_END    [B, N, N, H, D], index [b, j, i, h, c]: the same pair layout,
 *                               attending along the first pair index with the second one fixed
 *                               (ending node), with no transposed copy
 *
 * AlphaFold3-style Pairformers, the models TurboPairFormer's kernel serves (Abstract), run
 * triangle attention around both the starting and the ending node; the ending-node form is
 * the starting-node form applied to the transposed pair representation.  Only addressing
 * changes with the layout: bias, dbias, key_mask and lse keep their layouts, indexed by slice
 * and by the tokens along the attended axis, so the ending-node caller passes the pair bias
 * and key mask for that orientation (N*N values per batch, not N*N*N).  For the same values in
 * either layout every output is bitwise identical.
 */
typedef enum {
  TRI_ATTN_LAYOUT_SLICE_HEAD = 0,
  TRI_ATTN_LAYOUT_PAIR_START = 1,
  TRI_ATTN_LAYOUT_PAIR_END = 2
} tri_attn_layout;

/*
 * Staged calls with an explicit token layout (an int holding a tri_attn_layout value);
 * tri_attn_fwd_stages / tri_attn_bwd_stages are these with TRI_ATTN_LAYOUT_SLICE_HEAD.
 * Errors beyond those of the staged calls: TRI_ATTN_ERROR_INVALID_VALUE for an unknown
 * layout; TRI_ATTN_ERROR_UNSUPPORTED when a slice's rows, padded to a multiple of 128 tokens,
 * span more than 2^31 - 1 bytes (PAIR_END with N*N*H*D*2 near 2 GiB; the kernels address a
 * slice with 32-bit offsets).
 */
tri_attn_status tri_attn_fwd_ex(unsigned stages, int layout, int64_t B, int64_t N, int64_t H, int64_t D,
                                const void *q, const void *k, const void *v, const void *bias,
                                const uint8_t *key_mask,
                                void *o, float *lse, void *residual,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

tri_attn_status tri_attn_bwd_ex(unsigned stages, int layout, int64_t B, int64_t N, int64_t H, int64_t D,
                                const void *q, const void *k, const void *v, const void *bias,
                                const uint8_t *key_mask,
                                const void *o, const float *lse, const void *residual,
                                const void *dO,
                                void *dq, void *dk, void *dv, float *dbias,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory while they run: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The same computation and results as tri_attn_fwd on the same arguments (same kernels, bit for
 * bit), without a workspace argument: the scratch it needs (B*H*ceil(N/64)*64*ceil(N/128)*128*4
 * bytes of prepared bias tiles, rounded up to 256) lives in a device array inside the library,
 * TRI_ATTN_NOALLOC_SCRATCH_BYTES = 64 MiB per GPU, which each GPU the library runs on holds
 * until the process ends.  The call makes no hipMalloc, hipFree or other allocating call.
 *   - Shapes needing more scratch than that return TRI_ATTN_ERROR_SCRATCH_LIMIT before anything
 *     is launched (at N = 768, up to B*H = 28 slices' heads fit; tri_attn_noalloc_scratch_bytes()
 *     and tri_attn_fwd_workspace_bytes() give the two sizes).
 *   - Every call on one GPU uses that GPU's one array, on the caller's stream: calls that
 *     overlap on one GPU (other streams, other host threads) race and must be serialised by
 *     the caller.  Nothing needs clearing between calls: each call writes all the scratch it
 *     reads before reading it.
 *   - The scratch belongs to the current device (hipGetDevice); `stream` must be a stream of
 *     that device.  Its address is looked up once per device, on the first call there.
 *   - Otherwise as tri_attn_fwd: slice-major layout [B, N, H, N, D], same validation and errors.
 */
#define TRI_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

size_t tri_attn_noalloc_scratch_bytes(void);

tri_attn_status tri_attn_fwd_noalloc(int64_t B, int64_t N, int64_t H, int64_t D,
                                     const void *q, const void *k, const void *v, const void *bias,
                                     const uint8_t *key_mask,
                                     void *o, float *lse, void *residual, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTN_H */
