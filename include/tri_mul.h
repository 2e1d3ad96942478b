/*
 * tri_mul.h — C ABI of the triangular multiplicative update in libtri_attn.so
 * (MI355X, gfx950).
 *
 * The pages name triangle multiplication as the other pair operation of the
 * AlphaFold-family stack, implemented with kernels of its own next to triangle
 * attention (TurboPairFormer news item, "Dove si impiega il tempo" and
 * "Benchmark di addestramento").  They do not write it out; the operation
 * taken is the update of the AlphaFold family as OpenFold3's Pairformer uses
 * it (linear layers without biases).  For every pair (i, j) of z [n][n][c_z]:
 *
 *   x      = LayerNorm(z)                        over c_z, gamma_in / beta_in
 *   a      = sigmoid(x W_ag^T) * (x W_ap^T)      [c]
 *   b      = sigmoid(x W_bg^T) * (x W_bp^T)      [c]
 *   g      = sigmoid(x W_g^T)                    [c_z]
 *   t_ij   = sum_k a_ik * b_jk                   (outgoing edges, incoming = 0)
 *   t_ij   = sum_k a_ki * b_kj                   (incoming edges, incoming = 1)
 *   y_ij   = g * (LayerNorm(t_ij) W_o^T)         over c, gamma_out / beta_out
 *
 * The contraction over the third token k costs 2 n^3 c flops forward and
 * 4 n^3 c backward.  LayerNorms use the biased variance.
 *
 * Conventions (as in tri_attn.h): device pointers owned by the caller,
 * contiguous, 16-byte aligned (saved and workspace: 256-byte aligned);
 * validation before any launch, negative TRI_ATTN_* status on error, no
 * stream synchronisation, nothing allocated.  Compiled for dtype
 * TRI_ATTN_BF16 with c_z = c = 128 (TRI_ATTN_EUNSUPPORTED otherwise) and
 * 1 <= n <= 4096; accumulation and statistics are fp32.  Weights use the
 * (out, in) convention of a linear layer:
 *   w_in  [4c + c_z][c_z]: the rows of W_ap, W_ag, W_bp, W_bg (c rows each), then W_g;
 *   w_out [c_z][c].
 * gamma_in, beta_in [c_z]; gamma_out, beta_out [c].
 */
#ifndef TRI_MUL_H
#define TRI_MUL_H

#include "tri_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the buffer the forward fills and the backward reads (the
 * intermediates the backward needs: LayerNorm statistics and outputs, the
 * projections, the gated edge operands, t and the gate); 0 on bad args. */
size_t tri_mul_saved_size(int n, int cz, int c, int dtype);

/* Bytes of device workspace tri_mul_bwd needs (0 on bad args). */
size_t tri_mul_workspace_size(int n, int cz, int c, int dtype);

/* Forward.  z, y [n][n][c_z]; saved: at least tri_mul_saved_size bytes, kept
 * unchanged for tri_mul_bwd with the same weights and flags; 0 < ln_eps < 1. */
int tri_mul_fwd(int n, int cz, int c, int dtype, int incoming,
                const void *z, const void *ln_in_gamma, const void *ln_in_beta, const void *w_in,
                const void *ln_out_gamma, const void *ln_out_beta, const void *w_out, float ln_eps,
                void *y, void *saved, size_t saved_bytes, tri_attn_stream_t stream);

/* Backward.  dy [n][n][c_z] -> dz [n][n][c_z] and the parameter gradients
 * (same shapes as the parameters), overwritten.  The weight gradients are sums
 * over the pairs in fixed split order and the LayerNorm parameter gradients
 * sums of fixed per-block partials in block order, so repeated calls give
 * bit-identical results.  workspace: at least tri_mul_workspace_size bytes,
 * contents on entry ignored. */
int tri_mul_bwd(int n, int cz, int c, int dtype, int incoming,
                const void *z, const void *ln_in_gamma, const void *ln_in_beta, const void *w_in,
                const void *ln_out_gamma, const void *ln_out_beta, const void *w_out, float ln_eps,
                const void *saved, size_t saved_bytes, const void *dy,
                void *dz, void *dln_in_gamma, void *dln_in_beta, void *dw_in,
                void *dln_out_gamma, void *dln_out_beta, void *dw_out,
                void *workspace, size_t workspace_bytes, tri_attn_stream_t stream);

/* tri_mul_fwd / tri_mul_bwd with stage timing, for benchmarks: identical
 * arguments and results, plus a non-NULL array of caller-created HIP events
 * (TRI_ATTN_EINVAL otherwise; NULL entries are not recorded) recorded on
 * `stream`.  Forward, 4 events: before the input side (LayerNorm, projections,
 * gating), before and after the contraction over the third token, after the
 * output side.  Backward, 5 events: before the output side's backward, before
 * the dA contraction (dA_c = dT_c B_c), between it and the dB contraction
 * (dB_c = dT_c^T A_c), after that, after the input side's backward. */
int tri_mul_fwd_profiled(int n, int cz, int c, int dtype, int incoming,
                         const void *z, const void *ln_in_gamma, const void *ln_in_beta, const void *w_in,
                         const void *ln_out_gamma, const void *ln_out_beta, const void *w_out, float ln_eps,
                         void *y, void *saved, size_t saved_bytes, tri_attn_stream_t stream,
                         tri_attn_event_t *events);
int tri_mul_bwd_profiled(int n, int cz, int c, int dtype, int incoming,
                         const void *z, const void *ln_in_gamma, const void *ln_in_beta, const void *w_in,
                         const void *ln_out_gamma, const void *ln_out_beta, const void *w_out, float ln_eps,
                         const void *saved, size_t saved_bytes, const void *dy,
                         void *dz, void *dln_in_gamma, void *dln_in_beta, void *dw_in,
                         void *dln_out_gamma, void *dln_out_beta, void *dw_out,
                         void *workspace, size_t workspace_bytes, tri_attn_stream_t stream,
                         tri_attn_event_t *events);

#ifdef __cplusplus
}
#endif

#endif /* TRI_MUL_H */
