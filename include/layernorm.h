/*
 * layernorm.h - LayerNorm entry points of the MI355X (gfx950) RMSNorm library.
 *
 * TransformerEngine PR #583 ("RMS Norm Optimization") registers matching
 * tuned configurations for LayerNorm beside RMSNorm and gives no formula.
 * The standard LayerNorm is implemented on the same kernels, with RMSNorm's
 * conventions (include/rmsnorm.h: storage types, eps and offset as float32
 * runtime scalars, the caller's stream, caller-owned buffers, fused residual
 * add, atomic-free dgamma partials and finalizer, argument checks before any
 * HIP call, rmsnorm_status codes and rmsnorm_last_error):
 *
 *   forward   mean_i = (1/N) sum_j v_ij
 *             rstd_i = 1 / sqrt((1/N) sum_j (v_ij - mean_i)^2 + eps)
 *             y_ij   = round_T((v_ij - mean_i) * rstd_i * (gamma_j + offset) + beta_j)
 *   backward  w_j = gamma_j + offset, g = dy * w, xhat = (v - mean_i) * rstd_i,
 *             dx_ij = round_T(rstd_i (g_ij - mean_j(g) - xhat_ij mean_j(g xhat)) [+ dh_ij])
 *             dgamma_j = round_T(sum_i dy_ij xhat_ij),  dbeta_j = round_T(sum_i dy_ij)
 *
 * gamma NULL means w_j = 1 (offset must be 0, dgamma NULL); beta NULL means
 * no bias (dbeta may still be asked for: it is the column sum of dy).
 */
#ifndef LAYERNORM_AMD_H
#define LAYERNORM_AMD_H

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* LayerNorm forward.
 *   x      [M, N] T     input rows
 *   gamma  [N] T        scale, used as gamma_j + offset (NULL: w = 1)
 *   beta   [N] T        bias (NULL: none)
 *   y      [M, N] T     output; may be NULL to compute the statistics only
 *   mean   [M] f32      saved row means for the backward (may be NULL)
 *   rstd   [M] f32      saved 1/std per row (may be NULL)
 * The 16-byte access path needs every pointer 16-byte aligned. */
int layernorm_fwd(const void *x, const void *gamma, const void *beta, void *y,
                  float *mean, float *rstd, int64_t M, int64_t N, float eps, float offset,
                  int dtype, rmsnorm_stream_t stream);

/* Fused residual add then LayerNorm: h_out receives round_T(x + residual)
 * (may alias residual) and the forward normalises that stored h. */
int layernorm_fused_add_fwd(const void *x, const void *residual, const void *gamma, const void *beta,
                            void *y, void *h_out, float *mean, float *rstd,
                            int64_t M, int64_t N, float eps, float offset,
                            int dtype, rmsnorm_stream_t stream);

/* Workspace the LayerNorm backward needs on the current device: two sets of
 * float32 partial rows (dgamma, dbeta) of programs x N (rows padded to 64
 * floats), plus 2 M floats used only when mean and rstd are not supplied. */
int layernorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, size_t *bytes);

/* LayerNorm backward: a bounded persistent grid writes dx and the dgamma and
 * dbeta partials into `workspace`; a finalizer sums each set in a fixed
 * order and writes dgamma and dbeta in T.  With up to four rows per program
 * (five on rows of more than 512 16-byte chunks; plan path
 * RMSNORM_PATH_ROWS_COLS) one launch does both: its first
 * workgroups write dx, the others sum dgamma_j = sum_i dy_ij * xhat_ij and
 * dbeta_j = sum_i dy_ij directly by columns in a fixed order, and the
 * workspace holds only recomputed mean and rstd.
 *   dy, x  [M, N] T;  gamma [N] T (NULL: w = 1, then dgamma NULL);
 *   mean, rstd [M] f32 from the forward, or both NULL to recompute them from x;
 *   dx     [M, N] T;  dgamma [N] T or NULL;  dbeta [N] T or NULL;
 *   workspace: at least layernorm_bwd_workspace_bytes() bytes, 16-byte
 *   aligned, contents ignored on entry and undefined on return.
 * M = 0 writes dgamma = dbeta = 0. */
int layernorm_bwd(const void *dy, const void *x, const void *gamma, const float *mean, const float *rstd,
                  void *dx, void *dgamma, void *dbeta, void *workspace, size_t workspace_bytes,
                  int64_t M, int64_t N, float eps, float offset,
                  int dtype, rmsnorm_stream_t stream);

/* Fused-add LayerNorm backward: h is the stored residual sum, dh the gradient
 * arriving at h_out (NULL for zero); dx = d(loss)/dx = d(loss)/dresidual and
 * may alias dh.  Other arguments as layernorm_bwd. */
int layernorm_fused_add_bwd(const void *dy, const void *dh, const void *h, const void *gamma,
                            const float *mean, const float *rstd, void *dx, void *dgamma, void *dbeta,
                            void *workspace, size_t workspace_bytes,
                            int64_t M, int64_t N, float eps, float offset,
                            int dtype, rmsnorm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LAYERNORM_AMD_H */
