/*
 * tri_mul.h — C ABI of the triangle multiplication core in libtriattn.so (gfx950, MI355X).
 *
 * The triangle multiplicative update of AlphaFold-family models lets each residue pair (i, j)
 * gather information through a third residue k, along the rows or the columns of the pair
 * representation, by elementwise gating, an outer product and a reduction over one index
 * (kongchang.com article on fast_trimul, section "什么是三角乘法更新").  TurboPairFormer
 * (arXiv 2610.05854, Abstract) runs triangle multiplication kernels next to its attention
 * kernel.  These entry points compute the cubic core of that update, for pair tensors a and
 * b that already carry their gating:
 *
 *   TRI_MUL_OUTGOING:  x[b,i,j,c] = sum_k a[b,i,k,c] * b[b,j,k,c]
 *   TRI_MUL_INCOMING:  x[b,i,j,c] = sum_k a[b,k,i,c] * b[b,k,j,c]
 *
 * and its gradients (x is bilinear in a and b):
 *
 *   OUTGOING:  da[i,k,c] = sum_j dx[i,j,c] b[j,k,c]     db[j,k,c] = sum_i dx[i,j,c] a[i,k,c]
 *   INCOMING:  da[k,i,c] = sum_j dx[i,j,c] b[k,j,c]     db[k,j,c] = sum_i dx[i,j,c] a[k,i,c]
 *
 * The projections, gating and normalisations around the core belong to the surrounding
 * module and are not part of these calls.
 *
 * Memory (caller-owned DEVICE memory, row-major, contiguous, 16-byte aligned), in one of two
 * layouts shared by all six tensors of a call:
 *   TRI_MUL_CHANNELS_LAST   bf16 [B, N, N, C], index [b, first pair index, second pair index, c]
 *                           (the layout of the pair representation); C a multiple of 8
 *   TRI_MUL_CHANNELS_FIRST  bf16 [B, C, N, N], index [b, c, first pair index, second pair index]
 *                           (each channel a plain N x N matrix); N a multiple of 8
 * The channels-first form is the fast one: every load is a run of contiguous elements of one
 * channel.  For the channels-last form there are two paths:
 *   - with a workspace (tri_mul_workspace_bytes, N a multiple of 8): the inputs are copied
 *     channels first into the workspace, the channels-first product runs, and the outputs are
 *     copied back (one extra read and write of each tensor);
 *   - without one (workspace NULL): a kernel that reads the pair layout in place, 8 channels
 *     per work-group, which spends most of each cache line it touches (several times slower).
 * Both paths, and the channels-first form, give bitwise-identical results on the same values.
 *
 * Arithmetic: bf16 products accumulated in FP32 on the matrix cores, one channel at a time;
 * each output is rounded once to bf16 (round to nearest even).  Every sum runs in a fixed
 * order that depends only on the shape: repeated calls give bitwise-identical outputs.
 *
 * Conventions: arguments are validated synchronously and nothing is launched on error; work
 * is enqueued on `stream`; outputs are overwritten and must not overlap the inputs; the
 * calls allocate nothing and need no workspace.
 */
#ifndef TRI_MUL_H
#define TRI_MUL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "tri_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TRI_MUL_OUTGOING = 0, /* reduce over the second pair index: rows i and j of the pair tensor */
  TRI_MUL_INCOMING = 1  /* reduce over the first pair index: columns i and j */
} tri_mul_direction;

typedef enum {
  TRI_MUL_CHANNELS_LAST = 0,
  TRI_MUL_CHANNELS_FIRST = 1
} tri_mul_layout;

/* Largest N accepted (element offsets inside one batch stay below 2^31 for C <= 1024). */
#define TRI_MUL_MAX_N 1024

/*
 * Bytes of device workspace for the fast channels-last path (the backward's five tensors
 * channels first); 0 for the channels-first layout, for N not a multiple of 8 (no fast path),
 * or for an invalid shape.  The same workspace serves the forward.  It is only valid for the
 * call it is passed to.
 */
size_t tri_mul_workspace_bytes(int layout, int64_t B, int64_t N, int64_t C);

/*
 * Forward: x from a and b.
 * Errors: TRI_ATTN_ERROR_INVALID_VALUE (NULL pointer, B/N/C < 1, unknown direction or layout,
 * x overlapping a or b); TRI_ATTN_ERROR_UNSUPPORTED (C > 1024, N > TRI_MUL_MAX_N, B > 2^16,
 * C not a multiple of 8 in the channels-last layout, N not a multiple of 8 in the
 * channels-first layout); TRI_ATTN_ERROR_MISALIGNED (a pointer not 16-byte aligned);
 * TRI_ATTN_ERROR_WORKSPACE (channels last, a workspace smaller than tri_mul_workspace_bytes);
 * TRI_ATTN_ERROR_LAUNCH.  workspace may be NULL (see the layouts above); it is ignored in the
 * channels-first layout and must not overlap any tensor.
 */
tri_attn_status tri_mul_fwd(int direction, int layout, int64_t B, int64_t N, int64_t C,
                            const void *a, const void *b, void *x,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward: da and db from a, b and the output gradient dx (same errors as tri_mul_fwd;
 * da and db must not overlap each other or the inputs).
 */
tri_attn_status tri_mul_bwd(int direction, int layout, int64_t B, int64_t N, int64_t C,
                            const void *a, const void *b, const void *dx, void *da, void *db,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Input gating of the update (the article's elementwise gating step; plainest reading as in
 * AlphaFold-family models): a = sigmoid(g) * p * mask[b, i, j], in FP32, rounded once to bf16.
 *   g, p     : bf16 [B, N, N, C], channels last (the layout projections of the pair
 *              representation produce); C a multiple of 8
 *   mask     : uint8 [B, N, N] (1 keep, 0 drop: the whole pair entry is zero), or NULL
 *   a        : bf16 in `layout`: channels last, or channels first [B, C, N, N] (N a multiple of
 *              8), so that the gated operand is written once, ready for the fast product
 * The backward takes da in the same layout and writes dg, dp channels last:
 *   dp = da * mask * sigmoid(g),   dg = da * mask * p * sigmoid(g) * (1 - sigmoid(g)).
 * Errors as for tri_mul_fwd (INVALID_VALUE also for an output overlapping an input).
 */
tri_attn_status tri_mul_gate_fwd(int layout, int64_t B, int64_t N, int64_t C,
                                 const void *g, const void *p, const uint8_t *mask, void *a,
                                 hipStream_t stream);

tri_attn_status tri_mul_gate_bwd(int layout, int64_t B, int64_t N, int64_t C,
                                 const void *g, const void *p, const uint8_t *mask, const void *da,
                                 void *dg, void *dp, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_MUL_H */
