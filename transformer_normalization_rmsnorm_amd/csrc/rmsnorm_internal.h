// Internal interfaces between the C ABI layer, the selector and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsnorm.h"

namespace rmsnorm {

// Launch geometry travels in the arguments: reading blockDim/gridDim inside a
// kernel costs a 16-bit vector load from the implicit arguments on gfx9,
// whose wait drains every outstanding load.
struct FwdArgs {
    const void *x;
    const void *r;     // residual (fused-add only)
    const void *gamma;
    void *y;           // may be null: rstd only
    void *h;           // fused-add output round(x + r)
    float *rstd;       // may be null
    int64_t M;
    int32_t N;
    float eps;
    float offset;
    int32_t threads = 0; // workgroup size of the launch
    int64_t grid = 0;    // workgroups of the launch
    // fp8 output only: y holds E4M3 codes of y * (*scale); each workgroup
    // writes max |y| to amax_part[blockIdx.x] when amax_part is not null
    const float *scale = nullptr;
    float *amax_part = nullptr;
    // LayerNorm only: bias (may be null) and the saved row means (may be null)
    const void *beta = nullptr;
    float *mean = nullptr;
};

struct BwdArgs {
    const void *dy;
    const void *v;     // x, or h for the fused-add op
    const void *gamma;
    const float *rstd;
    const void *dh;    // fused-add only (non-null)
    void *dx;
    float *partials;   // [programs, ld]
    int64_t ld;        // partial row stride in floats (multiple of 64)
    int64_t M;
    int32_t N;
    float offset;
    int32_t threads = 0; // workgroup size of the launch
    int64_t grid = 0;    // workgroups of the launch
    // LayerNorm only: the saved row means; the dbeta partials follow the
    // dgamma partials (program p's dbeta row at partials[(grid + p) * ld])
    const float *mean = nullptr;
    // One-launch backward (RMSNORM_PATH_ROWS_COLS, col_cs > 0): the
    // workgroups from `grid` on each own col_cs consecutive chunks of the row
    // and write dgamma (and for LayerNorm dbeta; T, either may be null)
    // directly; the row programs write no partial rows.
    void *dgamma = nullptr;
    void *dbeta = nullptr;
    int32_t col_cs = 0;
};

// Longest row accepted (2^24 elements).  Column and chunk indices, and the
// strided loop counters of the looped kernels, stay far inside int32 and the
// finalizer's launch inside HIP's 32-bit work-item count.
constexpr int64_t kMaxN = int64_t(1) << 24;

// Work-items of one launch are kept below 2^31; the row kernels stride over
// the rows, so capping the grid only makes them persistent.
constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

// Partial rows are padded to this many floats (256 bytes).
constexpr int64_t kPartialAlign = 64;
inline int64_t partial_ld(int64_t N) { return (N + kPartialAlign - 1) / kPartialAlign * kPartialAlign; }

// Finalizer geometry: each workgroup owns 32 columns (8 lanes x float4) and
// splits the partial rows over 32 groups of lanes.
constexpr int kFinThreads = 256;
constexpr int kFinColsPerBlock = 32;

// The compiled register-path configurations: X(vector access, team lanes
// (0 = whole workgroup), chunks per lane, rows loaded ahead).  This list is
// the one owner of "which kernels exist"; the selector and the dispatchers
// both expand it.
#define RMSNORM_FWD_ROWS_CONFIGS(X)                                                      \
    X(1, 8, 1, 0) X(1, 16, 1, 0) X(1, 32, 1, 0) X(1, 64, 1, 0) X(1, 64, 2, 0)            \
    X(1, 64, 4, 0) X(1, 0, 1, 0) X(1, 0, 2, 0) X(1, 0, 3, 0) X(1, 0, 4, 0) X(1, 0, 6, 0) \
    X(1, 0, 8, 0)                                                                        \
    X(1, 64, 8, 0) X(0, 64, 1, 0) X(0, 64, 2, 0) X(0, 64, 4, 0) X(0, 64, 8, 0)           \
    X(0, 0, 1, 0) X(0, 0, 2, 0) X(0, 0, 4, 0) X(0, 0, 8, 0) X(0, 0, 16, 0)               \
    X(1, 8, 1, 1) X(1, 16, 1, 1) X(1, 32, 1, 1) X(1, 16, 1, 2) X(1, 32, 1, 2)            \
    X(1, 64, 1, 1) X(1, 64, 2, 1) X(1, 64, 4, 1) X(1, 64, 8, 1) X(1, 64, 2, 2)          \
    X(1, 64, 4, 2)                                                                       \
    X(1, 0, 1, 1) X(1, 0, 2, 1) X(1, 0, 3, 1) X(1, 0, 4, 1) X(1, 0, 6, 1)                \
    X(1, 0, 1, 2) X(1, 0, 2, 2) X(1, 0, 3, 2) X(1, 0, 4, 2) X(1, 0, 1, 3) X(1, 0, 2, 3)

// Backward: X(vector access, team lanes, chunks per lane, rows loaded ahead,
// w in registers, launch bound, launch bound of the fused-add op).  With w in
// registers (1) each program loads w = gamma + offset once and keeps it for
// all its rows, the layout of FlyDSL PR #855 ("Hybrid atomic / two-stage
// backward"); with 0, gamma travels with every row through the cache instead,
// which frees 8 (bf16) or 4 (fp32) registers per chunk and lets rows of up to
// 32768 bf16 / 16384 fp32 elements stay in registers.  The launch bounds are
// the largest workgroups for which the entry compiles without spilling (1024
// threads: 128 VGPRs; 512: 256 VGPRs) in both dtypes; the fused-add op also
// holds the dh row.
#define RMSNORM_BWD_ROWS_CONFIGS(X)                                                      \
    X(1, 8, 1, 1, 1, 256, 256) X(1, 16, 1, 1, 1, 256, 256) X(1, 32, 1, 1, 1, 256, 256)   \
    X(1, 8, 1, 2, 1, 256, 256) X(1, 16, 1, 2, 1, 256, 256) X(1, 32, 1, 2, 1, 256, 256)   \
    X(1, 64, 1, 1, 1, 256, 256) X(1, 64, 2, 1, 1, 256, 256) X(1, 64, 1, 2, 1, 256, 256)  \
    X(1, 0, 1, 1, 1, 1024, 1024) X(1, 0, 1, 2, 1, 1024, 1024) X(1, 0, 1, 3, 1, 1024, 1024) \
    X(1, 0, 2, 0, 0, 1024, 1024) X(1, 0, 2, 1, 0, 1024, 1024) X(1, 0, 2, 2, 0, 512, 512) \
    X(1, 0, 3, 0, 0, 1024, 1024) X(1, 0, 3, 1, 0, 512, 512) X(1, 0, 4, 0, 0, 1024, 512)  \
    X(1, 0, 4, 1, 0, 512, 512) X(1, 0, 6, 0, 0, 512, 512) X(1, 0, 8, 0, 0, 512, 512)     \
    X(0, 64, 1, 1, 1, 256, 256) X(0, 64, 2, 1, 1, 256, 256) X(0, 0, 1, 1, 1, 1024, 1024) \
    X(0, 0, 2, 1, 1, 512, 512) X(0, 0, 4, 1, 1, 512, 512)

// LayerNorm backward: the same fields.  It also holds the row mean and a
// second set of accumulators (dbeta), so its bounds are its own.  The dbeta
// accumulators of workgroup teams with vector access live in LDS (N floats per
// workgroup) at four or more chunks per lane, and for the fused-add op, which
// also holds the dh row, at two or more (bwd_dbeta_in_lds).  A bound of 0: not
// compiled for that op.
#define RMSNORM_LN_BWD_ROWS_CONFIGS(X)                                                   \
    X(1, 8, 1, 1, 1, 256, 256) X(1, 16, 1, 1, 1, 256, 256) X(1, 32, 1, 1, 1, 256, 256)   \
    X(1, 64, 1, 1, 1, 256, 256) X(1, 64, 2, 1, 1, 256, 256)                              \
    X(1, 0, 1, 1, 1, 1024, 1024) X(1, 0, 1, 2, 1, 1024, 1024)                            \
    X(1, 0, 2, 0, 0, 1024, 1024) X(1, 0, 2, 1, 0, 1024, 1024) X(1, 0, 3, 0, 0, 1024, 1024) \
    X(1, 0, 4, 0, 0, 1024, 1024) X(1, 0, 4, 1, 0, 512, 512) X(1, 0, 6, 0, 0, 512, 512)   \
    X(1, 0, 8, 0, 0, 512, 512)                                                           \
    X(0, 64, 1, 1, 1, 256, 256) X(0, 64, 2, 1, 1, 256, 256) X(0, 0, 1, 1, 1, 1024, 1024) \
    X(0, 0, 2, 1, 1, 512, 512) X(0, 0, 4, 1, 1, 512, 512)

// Backward layouts that can reduce two rows together (rows_per_step = 2):
// RMSNorm (plain or fused-add) and plain LayerNorm (its two row sums for both
// rows in one four-sum reduction, up to 512 threads), workgroup teams, w in
// registers, one 16-byte chunk per lane, one step loaded ahead.  They run an instance of their own,
// whose depth template argument is kDepthPairs (no plan has that depth),
// compiled for up to bwd_pairs_bound(fused) threads.  The fused-add op also
// holds the dh rows (146 VGPRs); it is used up to 256 threads, where it
// measured faster (4096 x 2048 bf16 backward main 15.0 -> 14.1 us), and not
// at 512 (4096 x 4096: 24.2 against 24.4 us).
constexpr bool bwd_pairs_compiled(bool ln, bool fused, int team, int chunks, int depth, bool w_regs, int vec)
{
    return !(ln && fused) && team == 0 && chunks == 1 && depth == 1 && w_regs && vec > 1;
}
constexpr int bwd_pairs_bound(bool fused, bool ln = false) { return fused ? 256 : ln ? 512 : 1024; }
constexpr int kDepthPairs = 8;

// One-launch backward (RMSNORM_PATH_ROWS_COLS): the row layouts that have
// instances with column workgroups (workgroup teams of 16-byte chunks: one
// chunk per lane with w in registers, the layouts of rows of up to 1024
// chunks, or two with gamma re-read per row; RMSNorm and LayerNorm).
constexpr bool bwd_cols_layout(int team, int chunks, int w_regs, int vec)
{
    return team == 0 && vec > 1 && ((chunks == 1 && w_regs == 1) || (chunks == 2 && w_regs == 0));
}
// Column workgroups of a launch: one per col_cs chunks, rounded up to whole
// rounds over the 8 XCDs (the extra ones exit at once).
inline int64_t bwd_col_workgroups(int64_t nchunks, int col_cs)
{
    const int64_t ncol = (nchunks + col_cs - 1) / col_cs;
    return (ncol + 7) / 8 * 8;
}

// LayerNorm backward layouts with dbeta accumulated in LDS.
constexpr bool bwd_dbeta_in_lds(bool ln, bool fused, int team, int chunks, int vec)
{
    return ln && team == 0 && vec >= 4 && (chunks >= 4 || (fused && chunks >= 2));
}

// Which instances of a backward register layout exist.  A row tiled exactly
// (threads x chunks x vec == N) runs the instance without masking, a ragged
// row the masked one, which is also correct for exact rows.  Two bf16
// fused-add LayerNorm layouts fit their registers with only one of them: four
// chunks x 1024 threads (128 VGPRs) only unmasked, so the selector takes it
// only for exact tilings; eight chunks x 512 threads (256 VGPRs) only masked,
// which then runs exact rows as well.
enum BwdTiling { TILING_ANY = 0, TILING_EXACT_ONLY = 1, TILING_MASKED_ONLY = 2 };
constexpr int bwd_tiling(bool ln, bool fused, int elem_size, int vec, int team, int chunks, int bound)
{
    if (!(ln && fused && elem_size == 2 && vec > 1 && team == 0))
        return TILING_ANY;
    if (chunks == 4 && bound == 1024)
        return TILING_EXACT_ONLY;
    return chunks == 8 ? TILING_MASKED_ONLY : TILING_ANY;
}

// LayerNorm forward: the forward layouts without prefetch, up to this many
// chunks per lane (it also holds beta).
constexpr int kLnFwdMaxChunks = 8;

// Forward launch bound: teams of at most a wavefront run in 256-thread
// workgroups; a workgroup team holding more than two chunks per lane is capped
// at 512 threads so that it may use up to 256 VGPRs instead of spilling.
constexpr int fwd_rows_bound_rule(int team, int chunks)
{
    return team != 0 ? 256 : (chunks > 2 ? 512 : 1024);
}

// Launch bound of a compiled forward configuration, 0 if it is not compiled.
inline int fwd_rows_bound(bool vec, int team, int chunks, int depth)
{
#define RMSNORM_MATCH(V, TEAM, K, D)                                                     \
    if ((V) == (vec ? 1 : 0) && (TEAM) == team && (K) == chunks && (D) == depth)          \
        return fwd_rows_bound_rule(TEAM, K);
    RMSNORM_FWD_ROWS_CONFIGS(RMSNORM_MATCH)
#undef RMSNORM_MATCH
    return 0;
}

// Launch bound of a compiled backward configuration, 0 if it is not compiled.
inline int bwd_rows_bound(bool ln, bool fused, bool vec, int team, int chunks, int depth, int w_regs)
{
#define RMSNORM_MATCH(V, TEAM, K, D, WR, BOUND, FBOUND)                                  \
    if ((V) == (vec ? 1 : 0) && (TEAM) == team && (K) == chunks && (D) == depth &&        \
        (WR) == w_regs)                                                                   \
        return fused ? (FBOUND) : (BOUND);
    if (ln) {
        RMSNORM_LN_BWD_ROWS_CONFIGS(RMSNORM_MATCH)
    } else {
        RMSNORM_BWD_ROWS_CONFIGS(RMSNORM_MATCH)
    }
#undef RMSNORM_MATCH
    return 0;
}

// Storage dtypes the kernels are built for.
inline bool dtype_known(int dtype) { return dtype == RMSNORM_F32 || dtype == RMSNORM_BF16 || dtype == RMSNORM_F16; }
// Elements per 16-byte access, and bytes per element.
inline int vec_elems(int dtype) { return dtype == RMSNORM_F32 ? 4 : 8; }
inline int elem_bytes(int dtype) { return dtype == RMSNORM_F32 ? 4 : 2; }

// Selector (pure; selector.cpp).
int select_plan(int op, int64_t M, int64_t N, int dtype, bool vec_ok, int num_cus, rmsnorm_plan *out);
// Fill the derived fields (chunks, grid, programs, workspace, finalizer) of a
// plan whose path/vec/team/threads are set; returns false if it cannot run.
bool complete_plan(rmsnorm_plan *p, int64_t M, int64_t N, int dtype, int num_cus, bool keep_grid);
int64_t bwd_workspace_bytes(int64_t programs, int64_t M, int64_t N, bool ln);

// Ops with fp8 output (the forward with y in E4M3).
inline bool is_fp8_op(int op) { return op == RMSNORM_OP_FWD_FP8 || op == RMSNORM_OP_FUSED_ADD_FWD_FP8; }
// LayerNorm ops.
inline bool is_ln_op(int op) { return op >= RMSNORM_OP_LN_FWD && op <= RMSNORM_OP_LN_FUSED_ADD_BWD; }
inline bool is_bwd_op(int op)
{
    return op == RMSNORM_OP_BWD || op == RMSNORM_OP_FUSED_ADD_BWD || op == RMSNORM_OP_LN_BWD ||
           op == RMSNORM_OP_LN_FUSED_ADD_BWD;
}
inline bool is_fused_op(int op)
{
    return op == RMSNORM_OP_FUSED_ADD_FWD || op == RMSNORM_OP_FUSED_ADD_BWD || op == RMSNORM_OP_FUSED_ADD_FWD_FP8 ||
           op == RMSNORM_OP_LN_FUSED_ADD_FWD || op == RMSNORM_OP_LN_FUSED_ADD_BWD;
}

// Forward kernel families.
enum FwdKind { FWD_RMS = 0, FWD_RMS_FP8 = 1, FWD_LN = 2 };

// amax finalizer: one workgroup folds the per-workgroup maxima.
constexpr int kAmaxThreads = 1024;

// Kernel launchers (launch.hip), dispatching on the storage dtype to the
// per-type instances of the templates below (fwd_kernels.h, bwd_kernels.h,
// instantiated in fwd_<type>.hip and bwd_<type>.hip).  fp8: y is E4M3 (only
// the layouts without prefetch are compiled for it).
hipError_t launch_fwd(int dtype, bool fused, FwdKind kind, const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s);
hipError_t launch_amax_finalize(const float *part, int64_t programs, float *amax, hipStream_t s);
hipError_t launch_bwd(int dtype, bool fused, bool ln, const rmsnorm_plan &p, const BwdArgs &a, hipStream_t s);
// dgamma_j = sum_p partials[p * ld + j]; with dbeta (LayerNorm) also
// dbeta_j = sum_p partials[(programs + p) * ld + j].  Either output may be null.
hipError_t launch_finalize(int dtype, const float *partials, int64_t programs, int64_t ld, int64_t N,
                           void *dgamma, void *dbeta, hipStream_t s);

template <typename T>
hipError_t launch_fwd_typed(bool fused, FwdKind kind, const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s);
template <typename T>
hipError_t launch_bwd_typed(bool fused, bool ln, const rmsnorm_plan &p, const BwdArgs &a, hipStream_t s);
template <typename T>
hipError_t launch_finalize_typed(const float *partials, int64_t programs, int64_t ld, int64_t N, void *dgamma,
                                 void *dbeta, hipStream_t s);

} // namespace rmsnorm
