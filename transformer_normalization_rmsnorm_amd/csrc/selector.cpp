// Shape/dtype selector: a pure function from (op, M, N, dtype, alignment,
// compute-unit count) to a launch plan.  No HIP calls.
//
// Prior art it starts from (FlyDSL PR #855, "Runtime configuration and
// ownership" and "512-thread vec8 fast path"): a vector path for 16-byte
// aligned rows with N a multiple of the vector width, a scalar path otherwise,
// a persistent backward grid of about one to two programs per compute unit
// capped by the row count, and one owner for the vector/scalar decision.  Here
// that owner is the configuration table in rmsnorm_internal.h.  Narrow rows
// (up to 32 vectors) are shared by teams of 8-32 lanes so a wavefront holds
// several rows, and rows too wide for registers take the looped path.
#include <algorithm>
#include <cmath>

#include "rmsnorm_internal.h"

namespace rmsnorm {

namespace {

constexpr int kRowsThreads = 256;   // workgroup size when a team is at most one wavefront
constexpr int kLoopThreads = 1024;  // looped path workgroup size
constexpr int kBwdProgramsPerCU = 1; // persistent backward workgroup teams per compute unit
constexpr int kBwdTeamsPerCU = 2;    // persistent backward workgroups per compute unit (sub-wave teams)
constexpr int64_t kDeepRowsPerProgram = 32; // backward rows per program from which two rows are in flight
// fused-add backward: from this many rows per program, workgroups of at least
// kFusedHalfMinThreads with one chunk per lane and w in registers take half
// the lanes with two chunks each and gamma re-read per row
constexpr int64_t kFusedHalfRowsPerProgram = 8;
constexpr int kFusedHalfMinThreads = 896;
// Workgroups of at most this many threads reduce two rows together wherever
// the layout allows (bwd_pairs_compiled), ahead of two rows in flight one at
// a time.  Measured on MI355X, bf16 backward main, one row / two rows in
// flight / two rows per reduction: 256 threads 16384 x 2048 45.6 / 41.5 /
// 34.9 us, 1024 x 2048 5.5 / 5.7 / 5.1 us; 512 threads 4096 x 4096 19.5 / 19.2
// / 19.1 us, 16384 x 4096 65.5 / 64.6 / 64.3 us; but 1024 threads 4096 x 8192
// 35.5 / 36.5 / 38.7 us and 2048 x 8192 19.7 / - / 23.0 us.  The fused-add op
// (which also holds dh) gained at 256 threads (4096 x 2048: 14.9 -> 13.8 us)
// and not at 512 (4096 x 4096: 24.0 / 24.0 us).
constexpr int kPairMaxThreads = 512;
constexpr int kPairMaxThreadsFused = 256;
// Plain LayerNorm (two sums per row, so four per step): at 256 threads 4096 x
// 2048 bf16 18.6 -> 16.7 us, 16384 x 2048 49.1 -> 42.2 us, fp32 4096 x 1024
// 17.3 -> 15.4 us; at 512 threads within 2% either way (4096 x 4096 24.3 /
// 24.0 us, 16384 x 4096 68.3 / 69.9 us), so it stops at 256.
constexpr int kPairMaxThreadsLN = 256;
// One-launch backward (RMSNORM_PATH_ROWS_COLS) for few rows.  Its column
// workgroups read dy and x a second time; its row programs load the rows
// through the cache, so that read mostly finds them there.  Measured on
// MI355X against the two-stage backward at the same layout (cold buffers,
// bf16 unless noted), RMSNorm: one row per program 27-39% faster (64 x 2048
// 7.53 -> 5.35 us, 128 x 8192 -39%, 256 x 4096 -35%, 256 x 8192 -27%, fp32
// 128 x 2048 -29%, fused-add 256 x 2048 -34%); two rows 13-27% (512 x 2048
// -27%, 512 x 4096 -23%, 512 x 8192 -15%, fp32 512 x 4096 -13%, fused-add
// 512 x 4096 -16%); three 768 x 2048 -16%, 768 x 4096 -17%, fp32 768 x 2048
// -18%, but 768 x 8192 (12 MiB) -0.8%; four 1024 x 2048 -10%, but
// 1024 x 4096 (8 MiB) +3% and 1024 x 8192 +13%; eight (2048 x 2048) +8%.
// So: up to two rows per program, or up to four while the rows hold at most
// kColsMaxBytes.
constexpr int64_t kColsMaxBytes = int64_t(6) << 20;
// LayerNorm's two-stage backward writes and sums two partial rows per
// program (dgamma and dbeta), so one launch pays off further: up to four rows
// per program at any width it covers (16 MiB of rows).  Measured: one row per
// program 256 x 4096 -33%; two 512 x 4096 -24%, 512 x 8192 -21%, fp32
// 512 x 4096 -15%; three 768 x 4096 -18%, 768 x 8192 -13%; four 1024 x 2048
// -11%, 1024 x 4096 -7%, 1024 x 8192 -3%, fp32 1024 x 2048 -8%, fused-add
// 1024 x 4096 -2%; six (1536 x 4096) +2%, eight (2048 x 2048) +7%.  Its
// column workgroups fold two sums with a wavefront each, so they need at
// least 128 threads.
constexpr int64_t kColsMaxRowsPerProgramLN = 4;
// Rows of more than 512 16-byte chunks (bf16 4097-8192, fp32 2049-4096
// wide): the one-chunk layout needs 1024 lanes, a whole compute unit, so the
// column workgroups can only start once the row programs are done.  With two
// chunks per lane, gamma re-read per row and 512 lanes, they run beside the
// row programs.  Measured on MI355X (one launch at 1024 lanes / at 512 lanes
// with two chunks, one row ahead; bf16 unless noted), RMSNorm: 256 x 8192
// 7.81 / 6.41 us, 512 x 8192 10.31 / 8.84, fp32 512 x 4096 9.49 / 8.57;
// against the two-stage backward 768 x 8192 13.96 / 12.42, fp32 768 x 4096
// 13.30 / 11.97, 1024 x 8192 15.63 / 15.25, but fp32 1024 x 4096 14.96 /
// 15.21 and 1536 x 8192 19.55 / 21.26; in a second run against the
// two-stage backward 1024 x 8192 15.67 / 15.54 and 1024 x 7168 14.42 /
// 14.92.  So RMSNorm rows of this width take one launch up to three rows per
// program.  With fewer rows
// than programs, or at 768 lanes, the compute units without a row program
// already take the column workgroups, and half the lanes cost RMSNorm time
// (128 x 8192 5.07 / 5.28 us, 300 x 6144 6.27 / 6.76): it takes them above
// 768 lanes (measured at 1024; at 896 the row program likewise leaves no
// room for a second workgroup of its size) from one row per program on.  LayerNorm, whose rows hold two
// sums, takes them from 768 lanes on: 512 x 8192 12.37 / 9.60, 768 x 8192
// 15.70 / 13.20, 1024 x 8192 19.10 / 16.34, 300 x 6144 8.49 / 7.25, 128 x
// 8192 5.95 / 5.88 (and the two-stage 1536 x 8192 23.45 / 22.27).  At 512
// chunks (bf16 4096) two chunks at 256 lanes gained only 4% (768 x 4096
// 8.05 / 7.75 us).
constexpr int kColsHalfLanesAbove = 512;
constexpr int kColsHalfLanesAboveRMS = 768;
// LayerNorm at half the lanes pays off up to five rows per program: against
// the two-stage backward 1280 x 8192 21.87 / 19.26 us, fused-add 25.56 /
// 23.15, fp32 1280 x 4096 19.34 / 18.71, 1280 x 6144 17.65 / 17.25; six
// 1536 x 8192 -5% but fp32 1536 x 4096 +1% and 1536 x 6144 +2.5%; eight
// (2048 x 8192) +3.6%.
constexpr int64_t kColsMaxRowsPerProgramLNHalf = 5;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
int pow2_at_least(int64_t v)
{
    int p = 1;
    while (p < v)
        p <<= 1;
    return p;
}

bool is_bwd(int op) { return is_bwd_op(op); }
bool is_fused(int op) { return is_fused_op(op); }

// Launch bound of a compiled configuration, 0 if it is not compiled (the
// forward has no w_regs variants: it is always 0 there).
int bound(int op, bool vec, int team, int k, int depth, int w_regs)
{
    if (is_bwd(op))
        return bwd_rows_bound(is_ln_op(op), is_fused(op), vec, team, k, depth, w_regs);
    // fp8 output and LayerNorm: the forward layouts without prefetch only
    if ((is_fp8_op(op) || is_ln_op(op)) && depth != 0)
        return 0;
    if (is_ln_op(op) && k > kLnFwdMaxChunks)
        return 0;
    return w_regs == 0 ? fwd_rows_bound(vec, team, k, depth) : 0;
}

// Smallest compiled chunk count >= need for (vec, team, depth, w_regs).
int pick_chunks(int op, bool vec, int team, int depth, int w_regs, int64_t need)
{
    for (int k = 1; k <= 16; ++k)
        if (k >= need && bound(op, vec, team, k, depth, w_regs) > 0)
            return k;
    return 0;
}

// Workgroup-wide team: the fewest chunks per lane whose thread count (a
// multiple of 64) fits the kernel's launch bound, preferring `cap` threads.
// The backward (scalar access here) prefers one chunk per lane: its registers
// also hold w, the dgamma accumulators and the rows in flight.
bool pick_block_team(int op, bool vec, int64_t nchunks, int depth, rmsnorm_plan *p)
{
    const bool bwd = is_bwd(op);
    const int caps_fwd[2] = {512, 1024}, caps_bwd[2] = {1024, 1024};
    const int wr = bwd ? 1 : 0;
    for (int cap : bwd ? caps_bwd : caps_fwd) {
        for (int k = 1; k <= 16; ++k) {
            const int b = bound(op, vec, 0, k, depth, wr);
            if (b == 0)
                continue;
            const int64_t threads = std::max<int64_t>(64, round_up(ceil_div(nchunks, k), 64));
            if (threads <= cap && threads <= b) {
                p->team = 0;
                p->threads = (int32_t)threads;
                p->chunks = k;
                p->depth = depth;
                p->w_regs = wr;
                return true;
            }
        }
    }
    return false;
}

// Whether the compiled instances of a backward layout can run this tiling
// (bwd_tiling: some layouts exist only for rows tiled exactly).
bool tiling_ok(int op, int dtype, bool vec, int team, int k, int b, int64_t lanes, int64_t nchunks)
{
    const int t = bwd_tiling(is_ln_op(op), is_fused(op), elem_bytes(dtype), vec ? vec_elems(dtype) : 1, team, k, b);
    return t != TILING_EXACT_ONLY || lanes * k == nchunks;
}

// Backward rows too wide for w in registers: gamma is re-read with every row.
// The fewest chunks per lane whose thread count fits a compiled launch bound,
// with the deepest prefetch compiled at that size.
bool pick_wide_bwd_team(int op, int dtype, bool vec, int64_t nchunks, rmsnorm_plan *p)
{
    for (int k = 1; k <= 16; ++k) {
        const int64_t threads = std::max<int64_t>(64, round_up(ceil_div(nchunks, k), 64));
        for (int d = 3; d >= 0; --d) {
            const int b = bound(op, vec, 0, k, d, 0);
            if (b > 0 && threads <= b && tiling_ok(op, dtype, vec, 0, k, b, threads, nchunks)) {
                p->team = 0;
                p->threads = (int32_t)threads;
                p->chunks = k;
                p->depth = d;
                p->w_regs = 0;
                return true;
            }
        }
    }
    return false;
}

// ---- RMSNorm forward layout (plain and fused-add) -------------------------
//
// Chosen from a sweep on MI355X of every exact workgroup tiling compiled
// (threads = row vectors / chunks, a multiple of 64, within the launch bound)
// over N = 2048 ... 32768 and 2 ... 64 rows per compute unit, bf16 and fp32
// rows, plain and fused-add, cold rotating buffers, medians of 7 interleaved
// rounds.  Two regimes:
//   * from 16 rows per compute unit (several rounds of workgroups per unit,
//     so what one workgroup streams per unit time decides): two chunks per
//     lane where that tiling fits, else the fewest that fit.  Within 3% of the
//     fastest tiling at all but 5 of the 52 swept points of this regime, and
//     within 5.2% at those (fp32 12288 wide, fused 8192 / 16384 / 24576 wide);
//   * below (one round of workgroups, so one workgroup's latency decides): no
//     closed rule came within 15% of the fastest at every point, so the
//     chunks per lane measured fastest at the nearest swept (N, rows per unit)
//     are taken (kFwdLatency*), and the exact tiling with the nearest chunk
//     count is launched.
// LayerNorm and the fp8-output forward have their own tables (below).
struct FwdLatencyRow {
    int32_t n;
    int8_t k[3]; // chunks per lane at 2, 4, 8 rows per compute unit
};
constexpr FwdLatencyRow kFwdLatency16[] = {
    {2048, {2, 1, 1}},  {4096, {4, 2, 8}},  {6144, {1, 3, 6}},  {8192, {2, 8, 2}},
    {12288, {4, 8, 2}}, {16384, {4, 4, 2}}, {24576, {6, 6, 6}}, {32768, {8, 8, 8}},
};
constexpr FwdLatencyRow kFwdLatency16Fused[] = {
    {2048, {4, 2, 4}}, {4096, {8, 4, 8}}, {8192, {2, 8, 2}}, {16384, {8, 8, 2}}, {24576, {6, 6, 8}},
};
constexpr FwdLatencyRow kFwdLatency32[] = {
    {2048, {1, 4, 8}}, {4096, {4, 8, 8}}, {6144, {4, 8, 2}}, {8192, {8, 8, 2}}, {12288, {8, 6, 6}}, {16384, {8, 8, 8}},
};

// Exact workgroup tiling (threads = nchunks / k a multiple of 64 within the
// launch bound) with the compiled chunk count nearest `want` (log scale; ties
// to the smaller count).  Returns false if the row has no exact tiling.
bool pick_fwd_chunks(int op, bool vec, int64_t nchunks, int want, rmsnorm_plan *p)
{
    int best_k = 0;
    double best_d = 0.0;
    for (int k = 1; k <= 16; ++k) {
        const int b = bound(op, vec, 0, k, 0, 0);
        if (b == 0 || nchunks % k != 0)
            continue;
        const int64_t t = nchunks / k;
        if (t % 64 != 0 || t > b)
            continue;
        const double d = std::fabs(std::log2((double)k / (double)want));
        if (best_k == 0 || d < best_d - 1e-9) {
            best_k = k;
            best_d = d;
        }
    }
    if (best_k == 0)
        return false;
    p->team = 0;
    p->threads = (int32_t)(nchunks / best_k);
    p->chunks = best_k;
    p->depth = 0;
    p->w_regs = 0;
    return true;
}

// Fewest compiled chunks per lane, at least kmin, with an exact tiling.
bool pick_fwd_fewest(int op, bool vec, int64_t nchunks, int kmin, rmsnorm_plan *p)
{
    for (int k = kmin; k <= 16; ++k) {
        const int b = bound(op, vec, 0, k, 0, 0);
        if (b == 0 || nchunks % k != 0)
            continue;
        const int64_t t = nchunks / k;
        if (t % 64 == 0 && t <= b)
            return pick_fwd_chunks(op, vec, nchunks, k, p);
    }
    return false;
}

bool pick_fwd_rms_team(int op, int dtype, int64_t M, int64_t N, int64_t nchunks, int num_cus, rmsnorm_plan *p)
{
    const double rows_per_cu = (double)M / (double)std::max(num_cus, 1);
    // the nearest swept rows-per-unit bucket, on a log scale: 16 and up
    // (from 8 * sqrt(2) rows per unit) is the throughput regime
    if (rows_per_cu >= 8.0 * std::sqrt(2.0)) {
        if (pick_fwd_fewest(op, true, nchunks, 2, p) || pick_fwd_fewest(op, true, nchunks, 1, p))
            return true;
        return pick_block_team(op, true, nchunks, 0, p);
    }
    const int bucket = rows_per_cu < 2.0 * std::sqrt(2.0) ? 0 : rows_per_cu < 4.0 * std::sqrt(2.0) ? 1 : 2;
    const FwdLatencyRow *rows;
    size_t nrows;
    if (dtype == RMSNORM_F32) {
        rows = kFwdLatency32;
        nrows = sizeof kFwdLatency32 / sizeof kFwdLatency32[0];
    } else if (is_fused(op)) {
        rows = kFwdLatency16Fused;
        nrows = sizeof kFwdLatency16Fused / sizeof kFwdLatency16Fused[0];
    } else {
        rows = kFwdLatency16;
        nrows = sizeof kFwdLatency16 / sizeof kFwdLatency16[0];
    }
    size_t near = 0;
    for (size_t i = 1; i < nrows; ++i)
        if (std::fabs(std::log2((double)N / rows[i].n)) < std::fabs(std::log2((double)N / rows[near].n)))
            near = i;
    return pick_fwd_chunks(op, true, nchunks, rows[near].k[bucket], p) || pick_block_team(op, true, nchunks, 0, p);
}

// ---- LayerNorm and fp8-output forward layouts (plain and fused-add) -------
//
// Each chosen from a sweep on MI355X like the RMSNorm one (every exact
// workgroup tiling compiled, N = 2048 ... 32768 bf16 and 2048 ... 16384 fp32
// plain, 2048 ... 24576 bf16 fused-add, 2 ... 64 rows per compute unit, cold
// rotating buffers, medians of 3 interleaved rounds).  No rule on rows per
// unit alone came within 13% of the fastest at every point, and the previous
// fixed targets missed by up to 29% (LayerNorm: N / 16 threads, at least 256,
// e.g. 384 x 4 at 12288 bf16) and 33% (fp8: 256 threads, e.g. 256 x 1 at 2048
// bf16 with 64 rows per unit).  So the chunks per lane measured fastest at the
// nearest swept (N, rows per unit) are taken, preferring the neighbouring
// bucket's count within 1%; within 1% of the fastest tiling at every swept
// point of the sweep each table was built from.
struct FwdTableRow {
    int32_t n;
    int8_t k[6]; // chunks per lane at 2, 4, 8, 16, 32, 64 rows per compute unit
};
constexpr FwdTableRow kLnFwd16[] = {
    {2048, {2, 2, 2, 2, 4, 4}}, {4096, {2, 2, 8, 4, 4, 4}},  {6144, {3, 6, 4, 4, 6, 6}},
    {8192, {4, 8, 4, 4, 4, 4}}, {12288, {6, 8, 6, 6, 8, 8}}, {16384, {8, 8, 8, 8, 8, 8}},
    {24576, {6, 6, 6, 6, 6, 6}}, {32768, {8, 8, 8, 8, 8, 8}},
};
constexpr FwdTableRow kLnFwd16Fused[] = {
    {2048, {2, 2, 4, 4, 1, 1}},  {4096, {1, 2, 8, 2, 2, 1}},  {8192, {4, 8, 4, 4, 4, 1}},
    {16384, {8, 8, 8, 2, 2, 8}}, {24576, {6, 6, 6, 6, 6, 6}},
};
constexpr FwdTableRow kLnFwd32[] = {
    {2048, {2, 8, 8, 8, 8, 8}}, {4096, {4, 8, 8, 8, 8, 4}},  {6144, {8, 6, 2, 2, 2, 2}},
    {8192, {8, 8, 8, 8, 8, 2}}, {12288, {8, 6, 6, 6, 6, 6}}, {16384, {8, 8, 8, 8, 8, 8}},
};
constexpr FwdTableRow kF8Fwd16[] = {
    {2048, {2, 2, 4, 2, 2, 4}}, {4096, {2, 2, 2, 4, 8, 8}},  {6144, {4, 2, 3, 3, 3, 3}},
    {8192, {4, 4, 4, 4, 8, 8}}, {12288, {6, 8, 8, 8, 8, 8}}, {16384, {8, 8, 8, 8, 8, 8}},
    {24576, {8, 8, 8, 8, 8, 8}}, {32768, {8, 8, 8, 8, 8, 8}},
};
constexpr FwdTableRow kF8Fwd16Fused[] = {
    {2048, {4, 2, 4, 4, 4, 4}},  {4096, {2, 8, 8, 4, 2, 2}},  {8192, {2, 2, 2, 2, 2, 2}},
    {16384, {8, 2, 2, 2, 2, 2}}, {24576, {6, 6, 6, 6, 6, 6}},
};
constexpr FwdTableRow kF8Fwd32[] = {
    {2048, {4, 2, 8, 8, 8, 8}}, {4096, {4, 8, 4, 8, 8, 8}},  {6144, {6, 6, 6, 6, 6, 6}},
    {8192, {8, 8, 8, 8, 8, 8}}, {12288, {6, 6, 6, 6, 6, 6}}, {16384, {8, 8, 8, 8, 8, 8}},
};

template <size_t A, size_t B, size_t C>
bool pick_fwd_table(int op, int dtype, int64_t M, int64_t N, int64_t nchunks, int num_cus, const FwdTableRow (&t16)[A],
                    const FwdTableRow (&t16_fused)[B], const FwdTableRow (&t32)[C], rmsnorm_plan *p)
{
    const double rows_per_cu = (double)M / (double)std::max(num_cus, 1);
    // the nearest of 2, 4, ..., 64 rows per unit on a log scale
    const int bucket = rows_per_cu < 2.0 ? 0 : (int)std::min<long>(5, std::lround(std::log2(rows_per_cu)) - 1);
    const FwdTableRow *rows = dtype == RMSNORM_F32 ? t32 : is_fused(op) ? t16_fused : t16;
    const size_t nrows = dtype == RMSNORM_F32 ? C : is_fused(op) ? B : A;
    size_t near = 0;
    for (size_t i = 1; i < nrows; ++i)
        if (std::fabs(std::log2((double)N / rows[i].n)) < std::fabs(std::log2((double)N / rows[near].n)))
            near = i;
    return pick_fwd_chunks(op, true, nchunks, rows[near].k[bucket], p) || pick_block_team(op, true, nchunks, 0, p);
}

} // namespace

// Backward workspace: the partial rows (LayerNorm: dgamma's then dbeta's),
// then room for the row statistics recomputed when the caller has none
// (rstd; LayerNorm also the means).
int64_t bwd_workspace_bytes(int64_t programs, int64_t M, int64_t N, bool ln)
{
    const int64_t sets = ln ? 2 : 1;
    return round_up(sets * programs * partial_ld(N) * (int64_t)sizeof(float), 256) +
           sets * round_up(M * (int64_t)sizeof(float), 256);
}

bool complete_plan(rmsnorm_plan *p, int64_t M, int64_t N, int dtype, int num_cus, bool keep_grid)
{
    const bool bwd = is_bwd(p->op);
    const int VV = vec_elems(dtype);
    if (p->vec != 1 && p->vec != VV)
        return false;
    if (N % p->vec != 0)
        return false;
    if (p->threads < 64 || p->threads > 1024 || p->threads % 64 != 0)
        return false;
    const int64_t nchunks = N / p->vec;
    int64_t rows_per_block = 1;
    if (!bwd)
        p->w_regs = 0;
    if (p->rows_per_step <= 0)
        p->rows_per_step = 1;
    if (!bwd && p->rows_per_step != 1)
        return false;
    if (p->w_regs != 0 && p->w_regs != 1)
        return false;
    const bool cols = p->path == RMSNORM_PATH_ROWS_COLS;
    if (cols && (!bwd || p->team != 0 || p->vec == 1))
        return false;
    if (!cols)
        p->col_chunks = 0;
    if (p->path == RMSNORM_PATH_ROWS || cols) {
        if (p->team != 0) {
            if (p->team != 8 && p->team != 16 && p->team != 32 && p->team != 64)
                return false;
            if (p->threads % p->team != 0 || p->threads > 256)
                return false;
            rows_per_block = p->threads / p->team;
        }
        const int lanes = p->team ? p->team : p->threads;
        const int k = pick_chunks(p->op, p->vec != 1, p->team, p->depth, p->w_regs, ceil_div(nchunks, lanes));
        const int b = k == 0 ? 0 : bound(p->op, p->vec != 1, p->team, k, p->depth, p->w_regs);
        if (k == 0 || p->threads > b)
            return false;
        if (bwd && !tiling_ok(p->op, dtype, p->vec != 1, p->team, k, b, lanes, nchunks))
            return false;
        p->chunks = k;
        if (cols) {
            // (LayerNorm's column workgroups fold dgamma and dbeta with one
            // wavefront each)
            if (!bwd_cols_layout(p->team, k, p->w_regs, p->vec) || p->threads < (is_ln_op(p->op) ? 128 : 64))
                return false;
            if (p->col_chunks <= 0) {
                // slab width: about one row per thread of a column workgroup
                // (threads / M) and about one column workgroup per compute
                // unit (nchunks / num_cus), the larger, as a power of two
                const int64_t want = std::max<int64_t>(ceil_div(p->threads, std::max<int64_t>(M, 1)),
                                                       ceil_div(nchunks, std::max(num_cus, 1)));
                p->col_chunks = (int32_t)std::min<int64_t>(8, pow2_at_least(want));
            }
            if (p->col_chunks != 1 && p->col_chunks != 2 && p->col_chunks != 4 && p->col_chunks != 8)
                return false;
        }
        if (p->rows_per_step != 1 &&
            (p->rows_per_step != 2 ||
             !bwd_pairs_compiled(is_ln_op(p->op), is_fused(p->op), p->team, k, p->depth, p->w_regs, p->vec) ||
             p->threads > bwd_pairs_bound(is_fused(p->op), is_ln_op(p->op))))
            return false;
        const int64_t sets = is_ln_op(p->op) ? 2 : 1;
        if (bwd && p->team != 0 && sets * rows_per_block * N * (int64_t)sizeof(float) > 65536)
            return false; // team partials are combined in LDS
    } else if (p->path == RMSNORM_PATH_LOOP) {
        if (p->rows_per_step != 1)
            return false;
        p->team = 0;
        p->chunks = 0;
        p->depth = 0;
        p->w_regs = 0;
    } else {
        return false;
    }
    const int64_t blocks_needed = std::max<int64_t>(1, ceil_div(M, rows_per_block));
    if (bwd) {
        const int per_cu = (p->path == RMSNORM_PATH_ROWS && p->team != 0) ? kBwdTeamsPerCU : kBwdProgramsPerCU;
        const int64_t want = keep_grid && p->grid > 0 ? p->grid : (int64_t)per_cu * std::max(num_cus, 1);
        p->grid = M == 0 ? 0 : std::min(want, blocks_needed);
        p->programs = cols ? 0 : p->grid;
        p->workspace_bytes = bwd_workspace_bytes(p->programs, M, N, is_ln_op(p->op));
        p->fin_threads = cols ? p->threads : kFinThreads;
        p->fin_grid = cols ? bwd_col_workgroups(nchunks, p->col_chunks)
                           : ceil_div(partial_ld(N), kFinColsPerBlock) * (is_ln_op(p->op) ? 2 : 1);
    } else {
        const int64_t want = keep_grid && p->grid > 0 ? p->grid : blocks_needed;
        p->grid = M == 0 ? 0 : std::min(std::min(want, blocks_needed), (kMaxWorkItems - 1) / p->threads);
        if (is_fp8_op(p->op)) { // one amax partial per workgroup
            p->programs = p->grid;
            p->workspace_bytes = round_up(std::max<int64_t>(p->grid, 1) * (int64_t)sizeof(float), 256);
            p->fin_threads = kAmaxThreads;
            p->fin_grid = 1;
        } else {
            p->programs = 0;
            p->workspace_bytes = 0;
            p->fin_threads = 0;
            p->fin_grid = 0;
        }
    }
    return true;
}

int select_plan(int op, int64_t M, int64_t N, int dtype, bool vec_ok, int num_cus, rmsnorm_plan *out)
{
    if (op < RMSNORM_OP_FWD || op > RMSNORM_OP_LN_FUSED_ADD_BWD)
        return RMSNORM_EINVAL;
    if (!dtype_known(dtype))
        return RMSNORM_EUNSUPPORTED;
    if (M < 0 || N <= 0 || N > kMaxN)
        return RMSNORM_EINVAL;
    const bool bwd = is_bwd(op);
    const int VV = vec_elems(dtype);
    rmsnorm_plan p = {};
    p.op = op;
    p.path = RMSNORM_PATH_ROWS;
    const bool vec = vec_ok && (N % VV == 0);
    p.vec = vec ? VV : 1;
    // forward: one row per team, no prefetch; backward: persistent, one row
    // ahead, w held in registers
    p.depth = bwd ? 1 : 0;
    p.w_regs = bwd ? 1 : 0;
    p.rows_per_step = 1;
    const int64_t nchunks = N / p.vec;
    bool placed = false;
    if (vec) {
        if (nchunks <= 32) {
            // narrow rows: several rows per wavefront
            p.team = std::max(8, pow2_at_least(nchunks));
            p.threads = kRowsThreads;
            placed = true;
        } else if (bwd && nchunks <= 128) {
            // one wavefront per row
            p.team = 64;
            p.threads = kRowsThreads;
            placed = true;
        } else {
            // backward: w in registers with one chunk per lane (the pages'
            // layout), else gamma re-read per row.  Measured on MI355X, gamma
            // per row with two chunks per lane and one row ahead beats w in
            // registers with three (bf16 8192 x 12288: 106.6 vs 109.3 us;
            // fp32 16384 x 6144: 197.3 vs 204.1 us) and ties it at 10240 bf16.
            if (bwd)
                placed = (nchunks <= 1024 && pick_block_team(op, true, nchunks, p.depth, &p)) ||
                         pick_wide_bwd_team(op, dtype, true, nchunks, &p);
            else if (is_fp8_op(op))
                placed = pick_fwd_table(op, dtype, M, N, nchunks, num_cus, kF8Fwd16, kF8Fwd16Fused, kF8Fwd32, &p);
            else if (is_ln_op(op))
                placed = pick_fwd_table(op, dtype, M, N, nchunks, num_cus, kLnFwd16, kLnFwd16Fused, kLnFwd32, &p);
            else
                placed = pick_fwd_rms_team(op, dtype, M, N, nchunks, num_cus, &p);
        }
    } else {
        if (nchunks <= (bwd ? 128 : 512)) {
            p.team = 64;
            p.threads = kRowsThreads;
            placed = true;
        } else {
            placed = pick_block_team(op, false, nchunks, p.depth, &p);
        }
    }
    if (!placed) {
        p.path = RMSNORM_PATH_LOOP;
        p.team = 0;
        p.threads = kLoopThreads;
    } else if (bwd && p.team == 0 && p.w_regs == 1 && !(is_ln_op(op) && is_fused(op))) {
        // Many rows per program: two rows in flight; with few, one (measured
        // on MI355X: 16384 x 8192 bf16 RMSNorm 138.3 -> 134.5 us and LayerNorm
        // 141.4 -> 136.3 us at two; 1024 x 8192, four rows per program, 16.0
        // against 16.9 us at one).  Fused-add LayerNorm, which also holds dh
        // and two accumulator sets, was 2.5% slower at two.
        const int64_t programs = (int64_t)kBwdProgramsPerCU * std::max(num_cus, 1);
        const int64_t rows = ceil_div(M, programs);
        if (rows >= 2 &&
            p.threads <= (is_fused(op) ? kPairMaxThreadsFused : is_ln_op(op) ? kPairMaxThreadsLN : kPairMaxThreads) &&
            bwd_pairs_compiled(is_ln_op(op), is_fused(op), p.team, p.chunks, p.depth, p.w_regs, p.vec) &&
            p.threads <= bwd_pairs_bound(is_fused(op), is_ln_op(op)))
            p.rows_per_step = 2;
        else if (is_fused(op) && p.chunks == 1 && p.threads >= kFusedHalfMinThreads &&
                 rows >= kFusedHalfRowsPerProgram && (p.threads / 2) % 64 == 0 &&
                 bound(op, vec, 0, 2, 1, 0) >= p.threads / 2 &&
                 tiling_ok(op, dtype, vec, 0, 2, bound(op, vec, 0, 2, 1, 0), p.threads / 2, nchunks)) {
            // The fused-add op also holds dh: at 896 or more lanes with w in
            // registers, half the lanes with two chunks each and gamma re-read
            // per row run faster once programs have several rows (sweep of the
            // backward layouts on MI355X, bf16 8192 wide at 8 to 64 rows per
            // compute unit 1-4.5%, fp32 4096 wide 1.4-2.9%; 16384 x 7168
            // bf16 148.9 against 157.1 us).  At 768 lanes or fewer it was not
            // faster.
            p.threads /= 2;
            p.chunks = 2;
            p.w_regs = 0;
            p.depth = 1;
        } else if (!is_fused(op) && rows >= kDeepRowsPerProgram && bound(op, vec, 0, p.chunks, 2, 1) >= p.threads)
            // (the fused-add op was 1.5-3.5% slower with two rows in flight in
            // the same sweep)
            p.depth = 2;
    } else if (bwd && p.team == 0 && p.w_regs == 0 && p.depth > 0) {
        // Wide rows (gamma re-read per row) with at most two rows per
        // program: no row ahead.  From sweeps of the backward layouts on
        // MI355X at 2 rows per compute unit, RMSNorm: fp32 8192 wide 13% and
        // 6144 wide 9% faster (fused-add 16% and 15%), bf16 fused-add 12288
        // and 16384 wide 7% and 10%, bf16 16384 wide 5%; LayerNorm: fp32
        // 6144 and 8192 wide 7% and 5% (fused-add 17% and 12%), bf16 fused-add
        // 12288 and 16384 wide 5% and 4%.  At four rows per program the plain
        // bf16 rows lost up to 7%, so the rule stops at two.
        const int64_t programs = (int64_t)kBwdProgramsPerCU * std::max(num_cus, 1);
        const int b0 = bound(op, vec, 0, p.chunks, 0, 0);
        if (ceil_div(M, programs) <= 2 && b0 >= p.threads &&
            tiling_ok(op, dtype, vec, 0, p.chunks, b0, p.threads, nchunks))
            p.depth = 0;
    }
    const bool ln = is_ln_op(op);
    if (placed && bwd && p.path == RMSNORM_PATH_ROWS && p.chunks == 1 &&
        bwd_cols_layout(p.team, p.chunks, p.w_regs, p.vec) && p.threads >= (ln ? 128 : 64) && M >= 1) {
        const int64_t programs = (int64_t)kBwdProgramsPerCU * std::max(num_cus, 1);
        const int64_t bytes = M * N * elem_bytes(dtype);
        // rows of more than 512 chunks: the row programs take two chunks per
        // lane with gamma re-read, at half the lanes (kColsHalfLanesAbove)
        const int b2 = bound(op, vec, 0, 2, 1, 0);
        const bool half = (ln ? p.threads > kColsHalfLanesAbove : (p.threads > kColsHalfLanesAboveRMS && M >= programs)) &&
                          (p.threads / 2) % 64 == 0 && b2 >= p.threads / 2 &&
                          tiling_ok(op, dtype, vec, 0, 2, b2, p.threads / 2, nchunks);
        const int64_t rms_rows = half ? 3 : 2;
        if (ln ? M <= (half ? kColsMaxRowsPerProgramLNHalf : kColsMaxRowsPerProgramLN) * programs
               : (M <= rms_rows * programs || (M <= 4 * programs && bytes <= kColsMaxBytes))) {
            p.path = RMSNORM_PATH_ROWS_COLS;
            p.col_chunks = 0; // the rule in complete_plan
            if (half) {
                p.threads /= 2;
                p.chunks = 2;
                p.w_regs = 0;
                p.depth = 1;
                p.rows_per_step = 1;
            }
        }
    }
    if (!complete_plan(&p, M, N, dtype, num_cus, false))
        return RMSNORM_EUNSUPPORTED;
    *out = p;
    return RMSNORM_OK;
}

} // namespace rmsnorm
