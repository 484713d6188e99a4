/*
 * rmsnorm.h - C ABI of the MI355X (gfx950) RMSNorm library.
 *
 * RMSNorm forward and backward, plain and with a fused residual add, for
 * bfloat16 and float32 storage with float32 arithmetic.
 *
 *   forward   rstd_i = 1 / sqrt((1/N) sum_j v_ij^2 + eps)
 *             y_ij   = round_T(v_ij * rstd_i * (gamma_j + offset))
 *   backward  w_j = gamma_j + offset, g = dy * w, xhat = v * rstd_i,
 *             c_i = (1/N) sum_j g_ij xhat_ij,
 *             dx_ij = round_T(rstd_i (g_ij - xhat_ij c_i) [+ dh_ij]),
 *             dgamma_j = round_T(sum_i dy_ij xhat_ij)
 *
 * Sources: Liger-Kernel PR #1388 "perf(cutedsl): add Blackwell fast path to
 * RMSNorm" (Summary; "1. TVM-FFI direct-call launch": eps and offset are
 * runtime float scalars, the caller's stream is used; "Results": "llama mode",
 * read as float32 compute with one cast after the gamma multiply) and ROCm/FlyDSL
 * PR #855 "[Perf] Optimize RMSNorm backward with staged reduction and vec8 I/O"
 * (Implementation: a bounded persistent backward grid writes dx and one float32
 * dgamma partial row per program, a finalizer reduces the [programs, N]
 * partials and writes dgamma in the parameter dtype with no atomics; fused-add
 * keeps the dx == dresidual aliasing contract; non-16-byte-aligned storage
 * offsets are supported; "Runtime configuration and ownership": the workspace
 * is per invocation and caller-owned, M is a runtime argument).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are device pointers on the current HIP device.  [M, N]
 *     tensors are contiguous and row-major (row stride N); gamma and dgamma
 *     are [N]; rstd is [M] float32.  Any element-aligned address is accepted;
 *     16-byte alignment of every pointer enables the 128-bit access path.
 *   - dtype: RMSNORM_BF16, RMSNORM_F16 or RMSNORM_F32 for every T-typed
 *     tensor of a call (FlyDSL PR #855, "512-thread vec8 fast path": the
 *     128-bit path serves FP16 and BF16, and its coverage list tests FP32,
 *     FP16 and BF16).  Arithmetic is float32 for every dtype; each T-typed
 *     output is rounded once, to nearest with ties to even.
 *   - Ownership: the caller owns every buffer, including the backward
 *     workspace.  The library allocates no device memory, keeps no per-call
 *     state, never synchronises, and launches only on `stream` (NULL = the
 *     null stream), so every call may be captured into a HIP graph.  Its only
 *     device memory is the fixed static scratch of rmsnorm_bwd_noalloc.
 *   - Errors: every function returns an rmsnorm_status.  All argument checks
 *     happen before any HIP call; a failed launch returns RMSNORM_EHIP.
 *     rmsnorm_last_error() gives a message for the calling thread's last
 *     failure.  Faults inside a kernel surface at the caller's next
 *     synchronisation, as for any asynchronous HIP work.
 *   - Aliasing: only h_out may alias residual (fused forward) and only dx may
 *     alias dh (fused backward); any other overlap is undefined.
 *   - M = 0 is valid: the forward does nothing; the backward writes
 *     dgamma = 0.  N must be in [1, 2^24] (RMSNORM_MAX_N).
 *   - gamma == NULL selects the non-affine op (no elementwise scale, w_j = 1;
 *     Liger-Kernel PR #1388 "Validation" covers affine and non-affine).  offset
 *     must then be 0 and dgamma NULL; the backward writes no partials, so it
 *     needs a workspace only to recompute rstd.
 *   - Results are deterministic: for a given device, shape, dtype and pointer
 *     alignment every output, dgamma included, is bit-identical run to run.
 */
#ifndef RMSNORM_AMD_H
#define RMSNORM_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type (hipStream_t is `struct ihipStream_t *`). */
struct ihipStream_t;
typedef struct ihipStream_t *rmsnorm_stream_t;

typedef enum rmsnorm_dtype {
    RMSNORM_F32 = 0,
    RMSNORM_BF16 = 1,
    RMSNORM_F16 = 2 /* IEEE binary16 */
} rmsnorm_dtype;

typedef enum rmsnorm_status {
    RMSNORM_OK = 0,
    RMSNORM_EINVAL = 1,       /* bad argument (null pointer, size, alignment, eps) */
    RMSNORM_EUNSUPPORTED = 2, /* dtype or configuration not available */
    RMSNORM_EWORKSPACE = 3,   /* workspace missing or smaller than required */
    RMSNORM_EHIP = 4          /* a HIP runtime call or kernel launch failed */
} rmsnorm_status;

/* Forward (Liger-Kernel PR #1388, Summary and "Results" llama mode; FlyDSL
 * PR #855 "Implementation": two-pass row math with a block reduction).
 *   x      [M, N] T   input rows
 *   gamma  [N] T      scale; the kernel uses gamma_j + offset (NULL: non-affine)
 *   y      [M, N] T   output, may be NULL to compute rstd only
 *   rstd   [M] f32    saved 1/rms per row for the backward, may be NULL
 *   eps >= 0 and offset: float32 runtime scalars. */
int rmsnorm_fwd(const void *x, const void *gamma, void *y, float *rstd,
                int64_t M, int64_t N, float eps, float offset,
                int dtype, rmsnorm_stream_t stream);

/* Fused residual add then forward (FlyDSL PR #855 "Hybrid atomic / two-stage
 * backward": fused-add is a specialization of the same op).
 *   h_out [M, N] T receives round_T(x + residual), computed in float32; the
 *   forward normalises that stored h.  h_out may alias residual.
 *   y may be NULL (h and rstd only); rstd may be NULL. */
int rmsnorm_fused_add_fwd(const void *x, const void *residual, const void *gamma,
                          void *y, void *h_out, float *rstd,
                          int64_t M, int64_t N, float eps, float offset,
                          int dtype, rmsnorm_stream_t stream);

/* Forward with float8 E4M3 output (TransformerEngine PR #583: the
 * normalization kernel's output type may be float8 E4M3, for its fp8 runs).
 * The page fixes only the type.  The readings follow the delayed-scaling use
 * of such an output:
 *   y_ij   = v_ij * rstd_i * (gamma_j + offset), in float32 as rmsnorm_fwd;
 *   y8_ij  = E4M3(y_ij * scale): OCP E4M3 "FN" (sign, 4 exponent bits with
 *            bias 7, 3 mantissa bits; largest finite 448; no infinities),
 *            nearest, ties to even, saturating at +-448;
 *   *amax  = max(*amax, max_ij |y_ij|), y before scaling, when amax != NULL.
 *   x      [M, N] T; gamma [N] T (NULL: non-affine)
 *   y8     [M, N] bytes, the E4M3 codes (required)
 *   rstd   [M] f32, may be NULL
 *   scale  device pointer to one float32 (read by the kernel, so a captured
 *          graph uses its value at replay)
 *   amax   device pointer to one float32, or NULL.  The caller initialises it
 *          (for example to 0) at the start of an amax window; each call folds
 *          its maximum in.  No atomics: every workgroup writes its maximum to
 *          `workspace` and a one-workgroup kernel folds them into *amax.
 *   workspace: needed only when amax != NULL: rmsnorm_fwd_fp8_workspace_bytes()
 *          bytes of device memory, 16-byte aligned, contents ignored on entry.
 * The 16-byte access path needs x, gamma 16-byte aligned and y8 aligned to
 * 16 / sizeof(T) bytes. */
int rmsnorm_fwd_fp8(const void *x, const void *gamma, void *y8, float *rstd,
                    const float *scale, float *amax, void *workspace, size_t workspace_bytes,
                    int64_t M, int64_t N, float eps, float offset,
                    int dtype, rmsnorm_stream_t stream);

/* Fused residual add then the fp8-output forward: h_out receives
 * round_T(x + residual) (may alias residual), y8/amax as rmsnorm_fwd_fp8 on h.
 * The 16-byte path also needs residual and h_out 16-byte aligned. */
int rmsnorm_fused_add_fwd_fp8(const void *x, const void *residual, const void *gamma,
                              void *y8, void *h_out, float *rstd,
                              const float *scale, float *amax, void *workspace, size_t workspace_bytes,
                              int64_t M, int64_t N, float eps, float offset,
                              int dtype, rmsnorm_stream_t stream);

/* Workspace the fp8-output forwards need when amax is requested: one float
 * per workgroup of the launch.  Writes the byte count to *bytes. */
int rmsnorm_fwd_fp8_workspace_bytes(int64_t M, int64_t N, int dtype, size_t *bytes);

/* Workspace the backward needs on the current device (FlyDSL PR #855
 * "Runtime configuration and ownership": programs * N * sizeof(float) of
 * partials, here with each partial row padded to 64 floats, plus M floats used
 * only when rstd is not supplied).  Writes the byte count to *bytes; depends
 * only on (M, N, dtype) and the device's compute-unit count. */
int rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, size_t *bytes);

/* Backward (FlyDSL PR #855 "Hybrid atomic / two-stage backward"): a bounded
 * persistent grid writes dx and float32 dgamma partials into `workspace`, then
 * a finalizer sums the partials in a fixed order and writes dgamma in T.
 * With few rows (up to two per program, four while the rows hold at most
 * 6 MiB, three on rows of more than 768 16-byte chunks; the plan's path is
 * then RMSNORM_PATH_ROWS_COLS) one launch does both:
 * its first workgroups write dx, the others sum
 * dgamma_j = sum_i dy_ij * x_ij * rstd_i directly by columns, in a fixed
 * order, and no partial rows are written.  Either way dgamma is
 * bit-identical run to run for the same shape, dtype and device.
 *   dy, x  [M, N] T;  gamma [N] T (NULL: non-affine, then dgamma NULL);
 *   rstd   [M] f32 from the forward, or NULL to recompute it from x with eps;
 *   dx     [M, N] T;  dgamma [N] T (NULL exactly when gamma is NULL);
 *   workspace: device memory of at least rmsnorm_bwd_workspace_bytes(), 16-byte
 *   aligned, contents ignored on entry and undefined on return. */
int rmsnorm_bwd(const void *dy, const void *x, const void *gamma, const float *rstd,
                void *dx, void *dgamma, void *workspace, size_t workspace_bytes,
                int64_t M, int64_t N, float eps, float offset,
                int dtype, rmsnorm_stream_t stream);

/* Fused-add backward (FlyDSL PR #855 "Fused-add RMSNorm backward": the
 * residual-gradient addition; "Hybrid ... backward": dx == dresidual).
 *   h   [M, N] T, the stored residual sum from rmsnorm_fused_add_fwd;
 *   dh  [M, N] T, gradient arriving at h_out, or NULL for zero;
 *   dx  [M, N] T = d(loss)/dx = d(loss)/dresidual; may alias dh (in place).
 *   Other arguments as rmsnorm_bwd (rstd NULL recomputes from h). */
int rmsnorm_fused_add_bwd(const void *dy, const void *dh, const void *h, const void *gamma,
                          const float *rstd, void *dx, void *dgamma,
                          void *workspace, size_t workspace_bytes,
                          int64_t M, int64_t N, float eps, float offset,
                          int dtype, rmsnorm_stream_t stream);

/* Backward that allocates nothing, for callers that cannot call hipMalloc or
 * hand over a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Arguments, results and checks are
 * rmsnorm_bwd's without the workspace; the dgamma partial rows (and rstd, when
 * it is recomputed) go to a library-owned static device buffer of
 * RMSNORM_NOALLOC_SCRATCH_BYTES on each device, held until the process ends.
 *   - A call whose workspace (rmsnorm_bwd_workspace_bytes, or its partial
 *     rows alone when rstd is given) exceeds that size returns
 *     RMSNORM_EWORKSPACE before any launch: at 256 compute units, rows up to
 *     16384 elements with rstd given.
 *   - Every call on a device shares that device's buffer, which keeps the last
 *     call's contents: calls that may overlap on one device (other streams,
 *     other threads) race and give undefined results.  Order them on one
 *     stream.
 *   - The first call on a device looks up the buffer's device address (no
 *     allocation); making that call outside graph capture is safest. */
#define RMSNORM_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int rmsnorm_bwd_noalloc(const void *dy, const void *x, const void *gamma, const float *rstd,
                        void *dx, void *dgamma, int64_t M, int64_t N, float eps, float offset,
                        int dtype, rmsnorm_stream_t stream);

/* The two backward stages on their own, for callers that reduce the dgamma
 * partials themselves (for example across devices, in rank order) and for
 * per-stage timing.
 *
 * rmsnorm_bwd_partials: dx as rmsnorm_bwd / rmsnorm_fused_add_bwd (dh NULL
 * for the plain op, v = x or h), and partials[p * ld + j] (float32, p <
 * *programs, j < N) with ld = N rounded up to a multiple of 64.  *programs
 * receives the number of partial rows written.  `workspace` is as for
 * rmsnorm_bwd; the partials are its first *programs * ld floats. */
int rmsnorm_bwd_partials(const void *dy, const void *v, const void *gamma, const float *rstd,
                         const void *dh, void *dx, void *workspace, size_t workspace_bytes,
                         int64_t *programs, int64_t M, int64_t N, float eps, float offset,
                         int dtype, rmsnorm_stream_t stream);

/* dgamma_j = round_T(sum_{p < programs} partials[p * ld + j]), summed in a
 * fixed order; ld = N rounded up to a multiple of 64; programs may be 0
 * (dgamma = 0).  partials must be 16-byte aligned. */
int rmsnorm_dgamma_finalize(const float *partials, int64_t programs, int64_t N,
                            void *dgamma, int dtype, rmsnorm_stream_t stream);

/* Launch plan chosen by the shape/dtype selector. */
typedef enum rmsnorm_op {
    RMSNORM_OP_FWD = 0,
    RMSNORM_OP_FUSED_ADD_FWD = 1,
    RMSNORM_OP_BWD = 2,
    RMSNORM_OP_FUSED_ADD_BWD = 3,
    RMSNORM_OP_FWD_FP8 = 4,
    RMSNORM_OP_FUSED_ADD_FWD_FP8 = 5,
    RMSNORM_OP_LN_FWD = 6,           /* LayerNorm (include/layernorm.h) */
    RMSNORM_OP_LN_FUSED_ADD_FWD = 7,
    RMSNORM_OP_LN_BWD = 8,
    RMSNORM_OP_LN_FUSED_ADD_BWD = 9
} rmsnorm_op;

typedef enum rmsnorm_path {
    RMSNORM_PATH_ROWS = 0, /* each row held in registers by a team of lanes */
    RMSNORM_PATH_LOOP = 1, /* rows streamed in passes (any N) */
    RMSNORM_PATH_ROWS_COLS = 2 /* backward with few rows: dx as on the ROWS path
                                  (workgroup teams, one chunk per lane with w in
                                  registers, or two with gamma re-read),
                                  and dgamma summed directly by fin_grid column workgroups
                                  of the same launch, each owning col_chunks consecutive
                                  chunks of the row over all rows: no partial rows and no
                                  second kernel */
} rmsnorm_path;

typedef struct rmsnorm_plan {
    int32_t op;          /* rmsnorm_op */
    int32_t path;        /* rmsnorm_path */
    int32_t vec;         /* elements per memory access: 16 / sizeof(T), or 1 */
    int32_t team;        /* lanes per row: 8, 16, 32, 64, or 0 = the whole workgroup */
    int32_t threads;     /* threads per workgroup of the main kernel */
    int32_t chunks;      /* vector accesses per lane per row and tensor (ROWS path) */
    int32_t depth;       /* rows a team loads ahead of the one it computes (ROWS path) */
    int32_t w_regs;      /* backward ROWS path: 1 = w = gamma + offset is loaded once per
                            program and held in registers; 0 = gamma is re-read with every
                            row (wide rows).  0 for the forward and the LOOP path. */
    int64_t grid;        /* workgroups of the main kernel (backward: row programs) */
    int64_t programs;    /* backward: dgamma partial rows (= grid; 0 on ROWS_COLS); fp8
                            forward: amax partials (= grid); plain forward: 0 */
    int64_t workspace_bytes; /* backward and fp8-forward workspace; plain forward 0 */
    int32_t fin_threads; /* finalizer workgroup size (dgamma, or amax for fp8) */
    int64_t fin_grid;    /* finalizer workgroups; ROWS_COLS: the column workgroups that
                            follow the grid row programs in the same launch */
    int32_t rows_per_step; /* backward ROWS path: rows a workgroup reduces together.  2: two
                              rows share one workgroup reduction and the next two are loaded
                              ahead (RMSNorm, plain or fused-add; workgroup teams, w in
                              registers, one chunk per lane, depth 1; at most 1024 threads,
                              256 for fused-add); otherwise 1. */
    int32_t col_chunks;  /* ROWS_COLS: 16-byte chunks of the row each column workgroup
                            sums over all rows (1, 2, 4 or 8); otherwise 0 */
} rmsnorm_plan;

/* Pure selector query: the plan for `op` at (M, N, dtype).  vec_ok != 0 says
 * every pointer of the call will be 16-byte aligned.  num_cus > 0 gives the
 * compute-unit count explicitly (no HIP call is made); num_cus <= 0 reads it
 * from the current device. */
int rmsnorm_query_plan(int op, int64_t M, int64_t N, int dtype, int vec_ok, int num_cus,
                       rmsnorm_plan *out);

/* Tuning and testing aid (the analogue of Liger-Kernel PR #1388's force
 * switches, "Behavior when the fast path does not apply"): later calls of `op`
 * use path, vec, team and threads from *plan, its depth and w_regs when they
 * are >= 0 and its grid when grid > 0 (else the selector's depth, w_regs and
 * grid for that layout), its rows_per_step when > 0 (else 1) and, on the
 * ROWS_COLS path, its col_chunks when > 0 (else the selector's rule); chunks
 * and the workspace follow.
 * vec = 1 forces scalar accesses on aligned data.  NULL clears.  Process-wide
 * and not thread-safe; a call that the override does not fit returns
 * RMSNORM_EINVAL. */
int rmsnorm_set_plan_override(int op, const rmsnorm_plan *plan);

const char *rmsnorm_status_string(int status);
const char *rmsnorm_last_error(void);
/* The ABI version this header describes (RMSNORM_ABI_VERSION); a binding
 * checks it before use.  2: rmsnorm_plan gained w_regs.  3: fp8-output
 * forwards (ops 4 and 5).  4: LayerNorm (include/layernorm.h, ops 6-9).
 * 5: binary16 storage (RMSNORM_F16).  6: rmsnorm_plan gained rows_per_step.
 * 7: rmsnorm_bwd_noalloc.  8: RMSNORM_PATH_ROWS_COLS; rmsnorm_plan gained
 * col_chunks. */
#define RMSNORM_ABI_VERSION 8

/* Longest row (elements) any entry point accepts. */
#define RMSNORM_MAX_N (1 << 24)
int rmsnorm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_AMD_H */
