/*
 * tri_attn.h — C ABI of the MI355X (gfx950) gated triangle self-attention
 * library (libtri_attn.so).
 *
 * The operation (starting node).  The pages describe it in words: a pair
 * representation attends, for each pair, over a third token, with a cost that
 * grows cubically in the token count (TurboPairFormer news item, section
 * "Dove si impiega il tempo"); the attention is gated (HelixFold review,
 * "Fused Gated Self-Attention"); the N^2 x N interaction map is computed tile
 * by tile in fast on-chip memory and never stored (MegaFold explainer,
 * EvoFlash-3D paragraph).  Written out:
 *
 *   s[i,h,j,k] = q[i,h,j,:].k[i,h,k,:] / sqrt(c) + bias[h,j,k]
 *                (-1e9 instead when mask[i,k] == 0)
 *   a[i,h,j,:] = sum_k softmax_k(s[i,h,j,:]) v[i,h,k,:]
 *   out[i,j,h,:] = sigmoid(gate[i,j,h,:]) * a[i,h,j,:]
 *
 * The backward recomputes each probability tile once and uses it for the
 * query, key, value and pair-bias gradients (TurboPairFormer news item, same
 * section); the pair-bias gradient is summed over rows i in a fixed order, so
 * repeated calls give bit-identical results (same item, "Accuratezza e
 * riproducibilità").
 *
 * Ending node (ending = 1): the same operation on the transposed pair layout,
 * end = T o start o T, where T swaps the two pair axes.  The caller keeps its
 * tensors in the ordinary pair layout; the kernels read and write them with the
 * pair axes swapped, so no transpose pass is made.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *    row-major, 16-byte aligned.  The library allocates nothing and keeps no
 *    state besides cached kernel attributes.
 *  - Element type of every tensor argument is `dtype` (TRI_ATTN_F32 or
 *    TRI_ATTN_BF16) except mask (uint8, nonzero = keep), lse (fp32) and the
 *    workspace (bytes).  bf16 runs accumulate in fp32.
 *  - Only c == 32 is compiled (TRI_ATTN_EUNSUPPORTED otherwise).
 *  - Rows: a call processes n_rows rows i (1 <= n_rows <= n) of an n x n pair
 *    representation.  Pointers point at the first processed row.  Starting
 *    node: q/k/v are [n_rows][h][n][c] and gate/out are [n_rows][n][h][c].
 *    Ending node: q/k/v are the caller's [n][h][n][c] tensors and gate/out are
 *    [n][n][h][c]; the processed rows i are along the SECOND pair axis, so the
 *    pointer for row i0 is base + i0*c (q/k/v) or base + i0*h*c (gate/out) and
 *    the mask pointer is base + i0.
 *  - bias is [h][n][n]: bias[h][j][k] (starting node, query j, key k); for the
 *    ending node the caller's bias[h][x][y] is read as bias[h][k][j].
 *  - attn_saved [n_rows][h][n][c] (dtype) and lse [n_rows][h][n] (fp32,
 *    natural-log log-sum-exp of each logit row) are written by the forward in
 *    kernel row order for both nodes and must be passed unchanged to the
 *    backward.
 *  - Validation happens before any launch: on an error nothing is launched and
 *    a negative status is returned.  Kernel launch failures return
 *    TRI_ATTN_EHIP.  No call synchronises the stream; device faults surface at
 *    the caller's next synchronisation.
 *  - Calls are reentrant; calls on different streams with different buffers
 *    may overlap.
 */
#ifndef TRI_ATTN_H
#define TRI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *tri_attn_stream_t; /* same object as hipStream_t */
typedef struct ihipEvent_t *tri_attn_event_t;   /* same object as hipEvent_t  */

enum { TRI_ATTN_F32 = 0, TRI_ATTN_BF16 = 1 };

enum {
  TRI_ATTN_OK = 0,
  TRI_ATTN_EINVAL = -1,       /* bad size, dtype, flag, null or misaligned pointer */
  TRI_ATTN_EUNSUPPORTED = -2, /* valid but not compiled (c != 32, n too large)    */
  TRI_ATTN_EWORKSPACE = -3,   /* workspace missing or smaller than required       */
  TRI_ATTN_EHIP = -4          /* a HIP call or kernel launch failed               */
};

/* Library version (major*10000 + minor*100 + patch). */
int tri_attn_version(void);

/* Static text for a status code; never NULL. */
const char *tri_attn_status_string(int status);

/* Largest n the compiled kernels accept for a dtype (0 for a bad dtype):
 * 2048 for bf16 (the forward's per-workgroup table of kept-key words), 736 for
 * fp32 (the fp32 backward past 256 keys keeps a row's K and V in LDS). */
int tri_attn_max_n(int dtype);

/* Bytes of device workspace tri_attn_fwd needs for these sizes (0 on bad args). */
size_t tri_attn_fwd_workspace_size(int n_rows, int n, int h, int c, int dtype);

/*
 * Forward pass.
 *   q, k, v     query/key/value, see conventions for the layout.
 *   bias        [h][n][n] pair bias (un-scaled; 1/sqrt(c) applies to q.k only).
 *   gate        gate pre-activation, same layout as out.
 *   mask        [n_rows][n] key mask for each row (row stride n, key stride 1;
 *               ending node: the caller's [n][n] mask read transposed), or NULL
 *               for "every key kept".  A row whose keys are all masked gets
 *               uniform weights over its n keys, as replacing every logit by
 *               the same constant implies.
 *   out         gated output.
 *   attn_saved  pre-gate attention a, kept for the backward.
 *   lse         log-sum-exp per logit row, kept for the backward.
 *   workspace   device scratch of at least tri_attn_fwd_workspace_size bytes,
 *               256-byte aligned (holds the bias tiles of this call in the
 *               order the kernel reads them).
 */
int tri_attn_fwd(int n_rows, int n, int h, int c, int dtype, int ending,
                 const void *q, const void *k, const void *v, const void *bias,
                 const void *gate, const uint8_t *mask,
                 void *out, void *attn_saved, float *lse,
                 void *workspace, size_t workspace_bytes, tri_attn_stream_t stream);

/*
 * tri_attn_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, layouts, results and errors are those of
 * tri_attn_fwd, bit for bit; the scratch the forward needs (the prepared bias
 * tiles, tri_attn_fwd_workspace_size bytes) comes from a fixed device array of
 * tri_attn_fwd_noalloc_max_bytes() bytes (16 MiB) inside the library, one per
 * device, held until the process ends.  Calls whose scratch would exceed it
 * return TRI_ATTN_EWORKSPACE before any device call (h = 4 fits up to
 * n = 1024).  The call allocates nothing: on the first call on a device it
 * looks up that device's copy of the array (TRI_ATTN_EHIP if that fails).
 * Every call on one device shares that device's array and leaves its contents
 * behind (the forward rewrites every byte it reads), so calls that overlap on
 * one device (different streams, different host threads without ordering)
 * race on it and must not be issued.
 */
int tri_attn_fwd_noalloc(int n_rows, int n, int h, int c, int dtype, int ending,
                         const void *q, const void *k, const void *v, const void *bias,
                         const void *gate, const uint8_t *mask,
                         void *out, void *attn_saved, float *lse, tri_attn_stream_t stream);

/* Size in bytes of tri_attn_fwd_noalloc's fixed scratch array. */
size_t tri_attn_fwd_noalloc_max_bytes(void);

/* Bytes of device workspace tri_attn_bwd needs for these sizes (0 on bad args).
 * The backward processes the call's rows in consecutive chunks of
 * tri_attn_bwd_chunk_rows rows that reuse one workspace (the gradient reaching
 * the pre-gate attention, the softmax row terms, and the partial sums of the
 * chunk's pair-bias and query gradients), so the workspace is bounded by the
 * chunk, not by n_rows: about 0.48 GB at n = n_rows = 768, h = 4, bf16. */
size_t tri_attn_bwd_workspace_size(int n_rows, int n, int h, int c, int dtype);

/* Rows per chunk of the backward for these sizes (0 on bad args); the call
 * runs ceil(n_rows / chunk) chunks.  The chunking does not change any result:
 * the pair-bias gradient is summed over rows in the same order as in one pass.
 * The library picks the chunk from a budget of about 300 MiB of partial sums;
 * the environment variable TRI_ATTN_BWD_CHUNK_ROWS (a positive integer, read on
 * every call of this function, tri_attn_bwd_workspace_size and the backward
 * entry points) replaces that choice, rounded down to whole 32-row blocks and
 * at least 32 rows; set it before sizing the workspace. */
int tri_attn_bwd_chunk_rows(int n_rows, int n, int h, int c, int dtype);

/*
 * Backward pass.  Inputs as for the forward plus attn_saved and lse from it and
 * dout (gradient of out, same layout as out).  Outputs, all in dtype:
 *   dq, dk, dv  same layouts as q, k, v.
 *   dbias       [h][n][n] (same reading as bias), summed over the n_rows rows
 *               of this call in ascending row-group order; overwritten.
 *   dgate       gradient w.r.t. the gate pre-activation, same layout as gate.
 * workspace     device scratch of at least tri_attn_bwd_workspace_size bytes,
 *               256-byte aligned; its contents on entry do not matter.
 * Results are bitwise identical across calls with the same inputs, sizes,
 * device and library build.
 */
int tri_attn_bwd(int n_rows, int n, int h, int c, int dtype, int ending,
                 const void *q, const void *k, const void *v, const void *bias,
                 const void *gate, const uint8_t *mask,
                 const void *attn_saved, const float *lse, const void *dout,
                 void *dq, void *dk, void *dv, void *dbias, void *dgate,
                 void *workspace, size_t workspace_bytes, tri_attn_stream_t stream);

/*
 * tri_attn_bwd with per-stage timing: identical arguments and results, plus
 * stage_events, an array of 4 caller-created HIP events per row chunk
 * (4 * ceil(n_rows / tri_attn_bwd_chunk_rows(...)) entries), recorded on
 * `stream`: for chunk m, entries 4m .. 4m+3 before its preprocessing, before
 * its main backward kernel, before its reductions (pair bias, query gradient)
 * and after them.  The preprocessing (gate gradient, D, the prepared bias
 * tiles) covers every row of the call in one pass before the first chunk, so
 * for later chunks entries 4m and 4m+1 mark the same point; only the fp32 path
 * past 256 keys preprocesses each chunk on its own.  A NULL entry is not recorded (each record puts a few
 * microseconds of idle time between the kernels it separates); the array
 * itself must be non-NULL (TRI_ATTN_EINVAL otherwise).  Intended for
 * benchmarks that need the main kernel's own duration.
 */
int tri_attn_bwd_profiled(int n_rows, int n, int h, int c, int dtype, int ending,
                          const void *q, const void *k, const void *v, const void *bias,
                          const void *gate, const uint8_t *mask,
                          const void *attn_saved, const float *lse, const void *dout,
                          void *dq, void *dk, void *dv, void *dbias, void *dgate,
                          void *workspace, size_t workspace_bytes, tri_attn_stream_t stream,
                          tri_attn_event_t *stage_events);

/* ------------------------------------------------------------------------
 * Rounding-residual compensation of the saved attention (bf16 only).
 *
 * The pages report that saving an approximation of the fp32 -> bf16 rounding
 * residual and using it in the backward, without changing the bf16 output,
 * lowers the error of the query, key and pair-bias gradients (TurboPairFormer
 * news item, "Accuratezza e riproducibilità").  Here the residual is that of
 * attn_saved: the forward writes, besides ab = bf16(a), one int8 code per
 * element,
 *
 *   code = clamp(round(256 * (a - ab) / u), -127, 127),   u = 2^(e - 134),
 *
 * where a is the fp32 attention value and e the biased exponent field of ab
 * (e = 1 for zero and subnormal ab; the code is 0 when ab is inf or NaN).
 * ab + code * u / 256 then equals a to within u / 512.  The backward
 * preprocessing uses that value for a in D = sum_c dA * a and in the gate
 * gradient; dq, dk and dbias depend on D, dv does not.
 *
 * attn_residual: int8 [n_rows][h][n][c], 16-byte aligned, written by
 * tri_attn_fwd_rc and passed unchanged to tri_attn_bwd_rc.  All other
 * arguments, results and errors are those of tri_attn_fwd / tri_attn_bwd;
 * dtype must be TRI_ATTN_BF16 and attn_residual non-NULL (TRI_ATTN_EINVAL
 * otherwise).
 * ------------------------------------------------------------------------ */
int tri_attn_fwd_rc(int n_rows, int n, int h, int c, int dtype, int ending,
                    const void *q, const void *k, const void *v, const void *bias,
                    const void *gate, const uint8_t *mask,
                    void *out, void *attn_saved, int8_t *attn_residual, float *lse,
                    void *workspace, size_t workspace_bytes, tri_attn_stream_t stream);

int tri_attn_bwd_rc(int n_rows, int n, int h, int c, int dtype, int ending,
                    const void *q, const void *k, const void *v, const void *bias,
                    const void *gate, const uint8_t *mask,
                    const void *attn_saved, const int8_t *attn_residual, const float *lse,
                    const void *dout, void *dq, void *dk, void *dv, void *dbias, void *dgate,
                    void *workspace, size_t workspace_bytes, tri_attn_stream_t stream);

/* ------------------------------------------------------------------------
 * The block around the attention: LayerNorm + projection front end and the
 * output linear, forward and backward.  The pages attribute the rest of the
 * pair stack's time to these LayerNorm and linear layers (TurboPairFormer news
 * item, "Dove si impiega il tempo"; ScaleFold summary, fused LayerNorm and
 * linear kernels) and fuse them into few passes (MegaFold explainer, EvoFusion
 * paragraph).  Written out, for every pair (a, b):
 *
 *   x_n   = (z[a,b,:] - mean) / sqrt(var + eps)     biased variance over c_z
 *   xhat  = x_n * gamma + beta
 *   q[a,h,b,:] | k | v | gate[a,b,h,:] = xhat . w_qkvg^T   (four blocks of h*c rows)
 *   bias[h,a,b] = xhat . w_bias[h,:]
 *   y[a,b,:] = out[a,b,:,:].flatten() . w_o^T
 *
 * The projections act on each pair alone, so the same calls serve the starting
 * and the ending node: tensors stay in the caller's pair layout and only the
 * attention call's `ending` flag differs.
 *
 * Compiled for dtype TRI_ATTN_BF16 with c_z = 128, c = 32, h*c = 128 only
 * (TRI_ATTN_EUNSUPPORTED otherwise); statistics are fp32, accumulation fp32.
 * Weights use the (out, in) convention of a linear layer: w_qkvg [4*h*c][c_z]
 * (rows: q as h*c + channel, then k, v, gate), w_bias [h][c_z], w_o [c_z][h*c].
 * Rows: a call processes pair rows a = 0..n_rows-1 of z [n_rows][n][c_z]; the
 * outputs q, k, v [n_rows][h][n][c], gate [n_rows][n][h][c] and the statistics
 * [n_rows][n] start at that slice; bias / dbias are addressed as
 * ptr[hh*n*n + a*n + b] (pass the full tensor's address + a0*n for a slice).
 * Alignment: 16 bytes for every tensor except bias, dbias, the weight and
 * LayerNorm gradients (2 bytes) and the statistics (4 bytes).
 * ------------------------------------------------------------------------ */

/* Front end forward: writes q, k, v, gate, bias and the LayerNorm statistics
 * ln_mean, ln_rstd (fp32, kept for the backward).  0 < ln_eps < 1. */
int tri_attn_ln_proj_fwd(int n_rows, int n, int cz, int h, int c, int dtype,
                         const void *z, const void *ln_gamma, const void *ln_beta, float ln_eps,
                         const void *w_qkvg, const void *w_bias,
                         void *q, void *k, void *v, void *gate, void *bias,
                         float *ln_mean, float *ln_rstd, tri_attn_stream_t stream);

/* Bytes of device workspace tri_attn_ln_proj_bwd needs (0 on bad args). */
size_t tri_attn_ln_proj_bwd_workspace_size(int n_rows, int n, int cz, int h, int c, int dtype);

/* Front end backward.  Inputs: z, gamma, beta, the saved statistics, the
 * weights and the gradients of the five projected tensors (dbias is the
 * complete gradient of bias, e.g. the attention backward's dbias).  Outputs
 * (overwritten): dz [n_rows][n][c_z]; dgamma, dbeta [c_z]; dw_qkvg, dw_bias,
 * each summed over this call's pairs in a fixed order (bitwise identical across
 * calls).  workspace: 256-byte aligned, contents on entry ignored. */
int tri_attn_ln_proj_bwd(int n_rows, int n, int cz, int h, int c, int dtype,
                         const void *z, const void *ln_gamma, const void *ln_beta,
                         const float *ln_mean, const float *ln_rstd,
                         const void *w_qkvg, const void *w_bias,
                         const void *dq, const void *dk, const void *dv, const void *dgate,
                         const void *dbias,
                         void *dz, void *dgamma, void *dbeta, void *dw_qkvg, void *dw_bias,
                         void *workspace, size_t workspace_bytes, tri_attn_stream_t stream);

/* Output linear forward: y [n_pairs][c_out] = x [n_pairs][c_in] . w^T, w [c_out][c_in]
 * (x is the attention output viewed as [pairs][h*c]).  c_in = c_out = 128. */
int tri_attn_out_proj_fwd(int n_pairs, int c_in, int c_out, int dtype,
                          const void *x, const void *w, void *y, tri_attn_stream_t stream);

/* Bytes of device workspace tri_attn_out_proj_bwd needs (0 on bad args). */
size_t tri_attn_out_proj_bwd_workspace_size(int n_pairs, int c_in, int c_out, int dtype);

/* Output linear backward: dx = dy . w; dw = dy^T . x summed over pairs in a
 * fixed order.  Outputs overwritten; workspace as above. */
int tri_attn_out_proj_bwd(int n_pairs, int c_in, int c_out, int dtype,
                          const void *x, const void *w, const void *dy,
                          void *dx, void *dw, void *workspace, size_t workspace_bytes,
                          tri_attn_stream_t stream);

/* ------------------------------------------------------------------------
 * Chunked inference of the starting-node block (forward only).  The FastFold
 * review ("提出的方法", "主要发现") describes memory-aware chunking for
 * inference, chosen automatically from the memory available.  Every step of
 * the block acts on one pair row i at a time except the pair bias, which each
 * row reads whole.  So the block can run over chunks of rows_per_chunk pair
 * rows, with only the bias and one chunk's intermediates resident:
 *
 *   pass 1, each chunk: LayerNorm + projections, keeping the bias rows;
 *   pass 2, each chunk: LayerNorm + projections again, attention over the full
 *   bias, output linear into the chunk's rows of y.
 *
 * y is bit for bit the y of the unchunked block
 * (tri_attn_ln_proj_fwd -> tri_attn_fwd -> tri_attn_out_proj_fwd) for every
 * rows_per_chunk; the projections are computed twice.  Sizes and dtypes are
 * those of the block calls (bf16, c_z = 128, h*c = 128); z, y [n][n][c_z]; mask
 * [n][n] or NULL; 1 <= rows_per_chunk <= n (TRI_ATTN_EINVAL otherwise).
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace for one rows_per_chunk (0 on bad args): the full
 * bias, one chunk's projections, attention outputs and statistics, and the
 * attention forward's workspace. */
size_t tri_attn_block_fwd_chunked_workspace_size(int n, int cz, int h, int c, int dtype, int rows_per_chunk);

/* The largest rows_per_chunk whose workspace fits in workspace_budget bytes,
 * or 0 when even one row does not fit (or the arguments are invalid). */
int tri_attn_block_chunk_rows(int n, int cz, int h, int c, int dtype, size_t workspace_budget);

/* The chunked forward: writes y.  workspace: 256-byte aligned, at least
 * tri_attn_block_fwd_chunked_workspace_size bytes, contents on entry ignored. */
int tri_attn_block_fwd_chunked(int n, int cz, int h, int c, int dtype, int rows_per_chunk,
                               const void *z, const void *ln_gamma, const void *ln_beta, float ln_eps,
                               const void *w_qkvg, const void *w_bias, const void *w_o,
                               const uint8_t *mask, void *y,
                               void *workspace, size_t workspace_bytes, tri_attn_stream_t stream);

/* ------------------------------------------------------------------------
 * Fused inference forward of the starting-node block.  The pages advocate
 * folding the front end (LayerNorm and the q / k / v / gate projections) into
 * the attention kernel (HelixFold review, "提出的方法": fused gated
 * self-attention; MegaFold explainer, EvoFusion paragraph).  This runs the
 * chunked forward's two passes with pass 2's front end split:
 *
 *   pass 1, each chunk: LayerNorm + pair-bias projection (as the chunked forward);
 *   pass 2, each chunk: LayerNorm + k / v projections only; then the attention
 *   kernel computes, in its prologue, LayerNorm and the q and gate projections
 *   of its own 32 queries per wave in registers (q and the gate never reach
 *   memory), runs the attention, applies the gate, and writes only the gated
 *   output (no saved attention, no log-sum-exp: there is no backward); output
 *   linear into the chunk's rows of y.
 *
 * y is bit for bit the y of tri_attn_block_fwd_chunked (and of the unchunked
 * block) for every rows_per_chunk: the fused prologue repeats the front end's
 * expressions and products.  Sizes, dtypes, layouts and errors as for
 * tri_attn_block_fwd_chunked.
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace (0 on bad args): the full bias, one chunk's k, v,
 * gated output and LayerNorm statistics, and the attention forward's workspace. */
size_t tri_attn_block_fwd_fused_workspace_size(int n, int cz, int h, int c, int dtype, int rows_per_chunk);

/* The fused forward: writes y.  workspace: 256-byte aligned, at least
 * tri_attn_block_fwd_fused_workspace_size bytes, contents on entry ignored. */
int tri_attn_block_fwd_fused(int n, int cz, int h, int c, int dtype, int rows_per_chunk,
                             const void *z, const void *ln_gamma, const void *ln_beta, float ln_eps,
                             const void *w_qkvg, const void *w_bias, const void *w_o,
                             const uint8_t *mask, void *y,
                             void *workspace, size_t workspace_bytes, tri_attn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTN_H */
