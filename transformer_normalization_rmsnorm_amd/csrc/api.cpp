// C ABI entry points: argument checks (before any HIP call), plan selection,
// launches on the caller's stream.  No allocation, synchronisation, copy or
// device-property query happens per call (the compute-unit count is read once
// per device), so every entry point can be captured into a HIP graph; that
// keeps small, host-bound shapes cheap (Liger-Kernel PR #1388, "Why the op was
// slow in the first place"; FlyDSL PR #855, "Hot-cache launch path").
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <tuple>

#include "layernorm.h"
#include "rmsnorm_internal.h"

using namespace rmsnorm;

static_assert(kMaxN == RMSNORM_MAX_N, "the header's row limit is the library's");

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

thread_local char g_err[512];

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_err[0] = '\0';
    return RMSNORM_OK;
}

// Test/tuning override per op.
struct Override {
    bool set = false;
    rmsnorm_plan plan = {};
};
Override g_override[10];

int device_cus(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(RMSNORM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(RMSNORM_EHIP, "device %d out of range", dev);
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || n <= 0)
            return fail(RMSNORM_EHIP, "compute-unit count of device %d: %s", dev, hipGetErrorString(e));
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    *cus = n;
    return RMSNORM_OK;
}

bool aligned(const void *p, size_t a) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(int64_t M, int64_t N, int dtype, float eps, float offset)
{
    if (!dtype_known(dtype))
        return fail(RMSNORM_EUNSUPPORTED, "dtype %d not supported (0 = f32, 1 = bf16, 2 = f16)", dtype);
    if (M < 0)
        return fail(RMSNORM_EINVAL, "M = %lld < 0", (long long)M);
    if (N <= 0 || N > kMaxN)
        return fail(RMSNORM_EINVAL, "N = %lld outside [1, 2^24]", (long long)N);
    if (M > 0 && M > INT64_MAX / N / 4)
        return fail(RMSNORM_EINVAL, "M * N too large");
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(RMSNORM_EINVAL, "eps must be finite and >= 0");
    if (!std::isfinite(offset))
        return fail(RMSNORM_EINVAL, "offset must be finite");
    return RMSNORM_OK;
}

// One-time plan log.  RMSNORM_LOG (read once, when the library is loaded; a
// value other than empty or "0" enables it) prints the plan a call takes, on
// stderr, once per (op, path, access width, dtype, N): the analogue of
// TransformerEngine PR #583's one-time warning with the type tuple when no
// tuned configuration exists ("Description").  The looped and per-element
// paths are such fallbacks here; their lines say so and why.
const bool g_log_plans = [] {
    const char *v = std::getenv("RMSNORM_LOG");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}();
std::mutex g_log_mu;
std::set<std::tuple<int, int, int, int, int64_t>> g_logged;

const char *op_name(int op)
{
    static const char *names[] = {"fwd", "fused_add_fwd", "bwd", "fused_add_bwd", "fwd_fp8", "fused_add_fwd_fp8",
                                  "ln_fwd", "ln_fused_add_fwd", "ln_bwd", "ln_fused_add_bwd"};
    return op >= 0 && op < 10 ? names[op] : "?";
}

const char *dtype_name(int dtype) { return dtype == RMSNORM_F32 ? "f32" : dtype == RMSNORM_BF16 ? "bf16" : "f16"; }

void log_plan(int op, int64_t M, int64_t N, int dtype, bool vec_ok, bool overridden, const rmsnorm_plan &p)
{
    {
        std::lock_guard<std::mutex> lock(g_log_mu);
        if (!g_logged.emplace(op, p.path, p.vec, dtype, N).second)
            return;
    }
    const bool per_elem = p.vec == 1;
    const char *why = "";
    if (p.path == RMSNORM_PATH_LOOP)
        why = per_elem ? " (fallback: looped rows, per-element access)" : " (fallback: looped rows, row too wide "
                                                                          "for the register layouts)";
    else if (per_elem)
        why = vec_ok ? " (fallback: per-element access, N not a multiple of the 16-byte vector)"
                     : " (fallback: per-element access, a pointer not 16-byte aligned)";
    std::fprintf(stderr,
                 "rmsnorm: %s %s N=%lld (first call M=%lld): path=%s vec=%d team=%d threads=%d chunks=%d depth=%d "
                 "w_regs=%d rows_per_step=%d grid=%lld workspace=%lld%s%s\n",
                 op_name(op), dtype_name(dtype), (long long)N, (long long)M,
                 p.path == RMSNORM_PATH_LOOP ? "loop" : p.path == RMSNORM_PATH_ROWS_COLS ? "rows+columns" : "rows", p.vec,
                 p.team, p.threads, p.chunks, p.depth, p.w_regs,
                 p.rows_per_step, (long long)p.grid, (long long)p.workspace_bytes, overridden ? " [override]" : "",
                 why);
}

// Plan for this call: the selector's, or the override's layout fitted to it.
int plan_for(int op, int64_t M, int64_t N, int dtype, bool vec_ok, int cus, rmsnorm_plan *p)
{
    int rc = select_plan(op, M, N, dtype, vec_ok, cus, p);
    if (rc != RMSNORM_OK)
        return fail(rc, "no plan for op %d M=%lld N=%lld dtype %d", op, (long long)M, (long long)N, dtype);
    const Override &o = g_override[op];
    if (o.set) {
        rmsnorm_plan q = *p;
        q.path = o.plan.path;
        q.vec = o.plan.vec;
        q.team = o.plan.team;
        q.threads = o.plan.threads;
        if (o.plan.depth >= 0)
            q.depth = o.plan.depth;
        if (o.plan.w_regs >= 0)
            q.w_regs = o.plan.w_regs;
        q.rows_per_step = o.plan.rows_per_step > 0 ? o.plan.rows_per_step : 1;
        q.col_chunks = o.plan.col_chunks;
        q.grid = o.plan.grid;
        if (q.vec != 1 && !vec_ok)
            return fail(RMSNORM_EINVAL, "override asks for 16-byte accesses on unaligned data");
        bool fits = complete_plan(&q, M, N, dtype, cus, true);
        if (!fits && o.plan.w_regs < 0) { // the selector's w_regs belongs to its own layout
            q.w_regs ^= 1;
            fits = complete_plan(&q, M, N, dtype, cus, true);
        }
        if (!fits)
            return fail(RMSNORM_EINVAL, "override plan does not fit M=%lld N=%lld", (long long)M, (long long)N);
        *p = q;
    }
    if (g_log_plans)
        log_plan(op, M, N, dtype, vec_ok, o.set, *p);
    return RMSNORM_OK;
}

int launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(RMSNORM_EHIP, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

// fp8 output (y holds E4M3 codes): the scale pointer, and the amax target
// with the workspace for its per-workgroup partials.
struct Fp8Out {
    const float *scale;
    float *amax;
    void *workspace;
    size_t workspace_bytes;
};

// LayerNorm forward extras: the bias (may be null) and the saved means.
struct LnFwd {
    const void *beta;
    float *mean;
};

int do_fwd(const void *x, const void *r, const void *gamma, void *y, void *h, float *rstd, int64_t M,
           int64_t N, float eps, float offset, int dtype, hipStream_t stream, bool fused,
           const Fp8Out *f8 = nullptr, const LnFwd *ln = nullptr)
{
    int rc = check_common(M, N, dtype, eps, offset);
    if (rc)
        return rc;
    if (f8 && (!y || !f8->scale))
        return fail(RMSNORM_EINVAL, "the fp8 forward needs y8 and scale");
    if (f8 && f8->amax && !aligned(f8->amax, 4))
        return fail(RMSNORM_EINVAL, "amax not aligned to 4 bytes");
    if (f8 && !aligned(f8->scale, 4))
        return fail(RMSNORM_EINVAL, "scale not aligned to 4 bytes");
    if (M == 0)
        return ok();
    if (!x || (fused && (!r || !h)))
        return fail(RMSNORM_EINVAL, "null input pointer");
    if (!gamma && offset != 0.0f)
        return fail(RMSNORM_EINVAL, "offset needs gamma (gamma == NULL is the non-affine op)");
    const void *beta = ln ? ln->beta : nullptr;
    float *mean = ln ? ln->mean : nullptr;
    if (!fused && !y && !rstd && !mean)
        return fail(RMSNORM_EINVAL, "no output requested: nothing to compute");
    const size_t eb = (size_t)elem_bytes(dtype);
    const size_t yb = f8 ? 1 : eb; // E4M3 codes are bytes
    if (!aligned(x, eb) || !aligned(gamma, eb) || !aligned(y, yb) || !aligned(r, eb) || !aligned(h, eb) ||
        !aligned(rstd, 4) || !aligned(beta, eb) || !aligned(mean, 4))
        return fail(RMSNORM_EINVAL, "pointer not aligned to its element size");
    if (y && (y == x || (gamma && y == gamma) || (beta && y == beta) || (fused && (y == r || y == h))))
        return fail(RMSNORM_EINVAL, "y aliases an input");
    if (fused && h == x)
        return fail(RMSNORM_EINVAL, "h_out aliases x (only residual may be overwritten)");
    // 16-byte accesses of T; the fp8 output then moves 16 / sizeof(T) bytes per access
    const size_t yv = f8 ? (size_t)vec_elems(dtype) : 16;
    const bool vec_ok = aligned(x, 16) && aligned(gamma, 16) && aligned(y, yv) && aligned(r, 16) &&
                        aligned(h, 16) && aligned(beta, 16);
    int cus = 0;
    if ((rc = device_cus(&cus)))
        return rc;
    const int op = ln ? (fused ? RMSNORM_OP_LN_FUSED_ADD_FWD : RMSNORM_OP_LN_FWD)
                 : f8 ? (fused ? RMSNORM_OP_FUSED_ADD_FWD_FP8 : RMSNORM_OP_FWD_FP8)
                      : (fused ? RMSNORM_OP_FUSED_ADD_FWD : RMSNORM_OP_FWD);
    rmsnorm_plan p;
    if ((rc = plan_for(op, M, N, dtype, vec_ok, cus, &p)))
        return rc;
    FwdArgs a{x, r, gamma, y, h, rstd, M, (int32_t)N, eps, offset};
    a.beta = beta;
    a.mean = mean;
    if (f8) {
        a.scale = f8->scale;
        if (f8->amax) {
            if (!f8->workspace || f8->workspace_bytes < (size_t)p.workspace_bytes)
                return fail(RMSNORM_EWORKSPACE, "workspace of %zu bytes given, %lld needed for amax",
                            f8->workspace ? f8->workspace_bytes : (size_t)0, (long long)p.workspace_bytes);
            if (!aligned(f8->workspace, 16))
                return fail(RMSNORM_EINVAL, "workspace not 16-byte aligned");
            a.amax_part = static_cast<float *>(f8->workspace);
        }
    }
    const FwdKind kind = ln ? FWD_LN : f8 ? FWD_RMS_FP8 : FWD_RMS;
    if ((rc = launched(launch_fwd(dtype, fused, kind, p, a, stream), "forward")))
        return rc;
    if (f8 && f8->amax)
        return launched(launch_amax_finalize(a.amax_part, p.programs, f8->amax, stream), "amax finalize");
    return ok();
}

// The two-stage layout a ROWS_COLS plan is built on (same rows layout and
// grid, partial rows and a finalizer).
bool two_stage(rmsnorm_plan *p, int64_t M, int64_t N, int dtype, int cus)
{
    rmsnorm_plan q = *p;
    q.path = RMSNORM_PATH_ROWS;
    q.col_chunks = 0;
    if (!complete_plan(&q, M, N, dtype, cus, true))
        return false;
    *p = q;
    return true;
}

// Shared by the backward entry points.  Writes dx and the partials; returns
// the number of partial rows in *programs.
// LayerNorm backward extras: the saved means (NULL together with rstd: both
// recomputed) and whether the partial rows (dgamma, dbeta) are wanted.
struct LnBwd {
    const float *mean;
    bool partials;
};

// The outputs a ROWS_COLS plan writes in the same launch as dx: dgamma (and
// for LayerNorm dbeta; either may be null); done is set when it did.
struct ColsOut {
    void *dgamma;
    void *dbeta;
    bool done;
};

// cols: the outputs of a full backward, which a ROWS_COLS plan writes in the
// same launch; NULL for the stage entry point, whose caller wants the partial
// rows, so such a plan runs as the two-stage layout it is built on.
int do_partials(const void *dy, const void *v, const void *gamma, const float *rstd, const void *dh, void *dx,
                void *workspace, size_t workspace_bytes, int64_t *programs, int64_t M, int64_t N, float eps,
                float offset, int dtype, hipStream_t stream, const LnBwd *ln = nullptr, ColsOut *cols = nullptr)
{
    int rc = check_common(M, N, dtype, eps, offset);
    if (rc)
        return rc;
    const bool fused = (dh != nullptr);
    const float *mean = ln ? ln->mean : nullptr;
    if (ln && ((mean == nullptr) != (rstd == nullptr)))
        return fail(RMSNORM_EINVAL, "mean and rstd must be given together (or both NULL to recompute)");
    if (!aligned(mean, 4))
        return fail(RMSNORM_EINVAL, "mean not aligned to 4 bytes");
    // partial rows: RMSNorm for dgamma (affine op); LayerNorm when dgamma or dbeta is wanted
    const bool want_partials = ln ? ln->partials : gamma != nullptr;
    if (M > 0 && (!dy || !v || !dx))
        return fail(RMSNORM_EINVAL, "null input pointer");
    if (!gamma && offset != 0.0f)
        return fail(RMSNORM_EINVAL, "offset needs gamma (gamma == NULL is the non-affine op)");
    const size_t eb = (size_t)elem_bytes(dtype);
    if (!aligned(dy, eb) || !aligned(v, eb) || !aligned(gamma, eb) || !aligned(dh, eb) || !aligned(dx, eb) ||
        !aligned(rstd, 4))
        return fail(RMSNORM_EINVAL, "pointer not aligned to its element size");
    if (!aligned(workspace, 16))
        return fail(RMSNORM_EINVAL, "workspace must be 16-byte aligned");
    if (M > 0 && (dx == dy || dx == v || (gamma && dx == gamma)))
        return fail(RMSNORM_EINVAL, "dx aliases an input other than dh");
    const bool vec_ok = aligned(dy, 16) && aligned(v, 16) && aligned(gamma, 16) && aligned(dh, 16) && aligned(dx, 16);
    int cus = 0;
    if ((rc = device_cus(&cus)))
        return rc;
    const int op = ln ? (fused ? RMSNORM_OP_LN_FUSED_ADD_BWD : RMSNORM_OP_LN_BWD)
                      : (fused ? RMSNORM_OP_FUSED_ADD_BWD : RMSNORM_OP_BWD);
    rmsnorm_plan p;
    if ((rc = plan_for(op, M, N, dtype, vec_ok, cus, &p)))
        return rc;
    if (p.path == RMSNORM_PATH_ROWS_COLS && (cols == nullptr || !want_partials) && !two_stage(&p, M, N, dtype, cus))
        return fail(RMSNORM_EINVAL, "no two-stage layout for this plan");
    // Workspace: the partial rows, then the recomputed row statistics (rstd;
    // LayerNorm: means, then rstd), M floats each, when the caller has none.
    const int64_t stat_region = ((M * 4 + 255) / 256) * 256;
    const int64_t stats = ln ? 2 : 1;
    const int64_t partial_region = p.workspace_bytes - stats * stat_region;
    const int64_t need = (want_partials ? partial_region : 0) + (rstd ? 0 : stats * stat_region);
    if (need > 0 && (workspace == nullptr || workspace_bytes < (size_t)need))
        return fail(RMSNORM_EWORKSPACE, "workspace of %zu bytes at %p; %lld bytes needed", workspace_bytes,
                    workspace, (long long)need);
    *programs = want_partials ? p.programs : 0;
    if (M == 0)
        return ok();
    const int64_t ld = partial_ld(N);
    float *partials = want_partials ? static_cast<float *>(workspace) : nullptr;
    const float *rs = rstd, *mu = mean;
    if (rs == nullptr) {
        // recompute the statistics from v into the workspace with a forward
        // that writes no y
        float *tail = reinterpret_cast<float *>(static_cast<char *>(workspace) + (want_partials ? partial_region : 0));
        float *tail_mu = ln ? tail : nullptr;
        float *tail_rs = ln ? reinterpret_cast<float *>(reinterpret_cast<char *>(tail) + stat_region) : tail;
        rmsnorm_plan fp;
        rc = select_plan(ln ? RMSNORM_OP_LN_FWD : RMSNORM_OP_FWD, M, N, dtype, aligned(v, 16) && aligned(gamma, 16),
                         cus, &fp);
        if (rc)
            return fail(rc, "no plan for the statistics recompute");
        FwdArgs fa{v, nullptr, gamma, nullptr, nullptr, tail_rs, M, (int32_t)N, eps, offset};
        fa.mean = tail_mu;
        if ((rc = launched(launch_fwd(dtype, false, ln ? FWD_LN : FWD_RMS, fp, fa, stream), "statistics recompute")))
            return rc;
        rs = tail_rs;
        mu = tail_mu;
    }
    BwdArgs a{dy, v, gamma, rs, dh, dx, partials, ld, M, (int32_t)N, offset};
    a.mean = mu;
    if (p.path == RMSNORM_PATH_ROWS_COLS) { // no partial rows: the column workgroups write the outputs
        a.partials = nullptr;
        a.dgamma = cols->dgamma;
        a.dbeta = cols->dbeta;
        a.col_cs = p.col_chunks;
        cols->done = true;
    }
    return launched(launch_bwd(dtype, fused, ln != nullptr, p, a, stream), "backward");
}

int do_finalize(const float *partials, int64_t programs, int64_t N, void *dgamma, int dtype, hipStream_t stream)
{
    if (!dtype_known(dtype))
        return fail(RMSNORM_EUNSUPPORTED, "dtype %d not supported", dtype);
    if (N <= 0 || N > kMaxN || programs < 0)
        return fail(RMSNORM_EINVAL, "bad N or programs");
    if (!dgamma || (programs > 0 && !partials))
        return fail(RMSNORM_EINVAL, "null pointer");
    if (!aligned(partials, 16) || !aligned(dgamma, (size_t)elem_bytes(dtype)))
        return fail(RMSNORM_EINVAL, "misaligned partials or dgamma");
    return launched(launch_finalize(dtype, partials, programs, partial_ld(N), N, dgamma, nullptr, stream),
                    "finalize");
}

// LayerNorm backward: dx and the partial rows, then dgamma and dbeta from a
// finalizer with one row of workgroups per output.
int do_ln_bwd(const void *dy, const void *dh, const void *v, const void *gamma, const float *mean,
              const float *rstd, void *dx, void *dgamma, void *dbeta, void *workspace, size_t workspace_bytes,
              int64_t M, int64_t N, float eps, float offset, int dtype, hipStream_t stream)
{
    if (!gamma && dgamma)
        return fail(RMSNORM_EINVAL, "dgamma given without gamma");
    if (dtype_known(dtype)) {
        const size_t eb = (size_t)elem_bytes(dtype);
        if (!aligned(dgamma, eb) || !aligned(dbeta, eb))
            return fail(RMSNORM_EINVAL, "dgamma or dbeta not aligned to its element size");
    }
    if (dbeta && (dbeta == dgamma || dbeta == dx))
        return fail(RMSNORM_EINVAL, "dbeta aliases another output");
    const LnBwd ln{mean, dgamma != nullptr || dbeta != nullptr};
    int64_t programs = 0;
    ColsOut cols{dgamma, dbeta, false};
    int rc = do_partials(dy, v, gamma, rstd, dh, dx, workspace, workspace_bytes, &programs, M, N, eps, offset,
                         dtype, stream, &ln, &cols);
    if (rc || !ln.partials || cols.done) // the one-launch backward has written dgamma and dbeta
        return rc;
    return launched(launch_finalize(dtype, static_cast<const float *>(workspace), programs, partial_ld(N), N,
                                    dgamma, dbeta, stream),
                    "finalize");
}

int do_bwd(const void *dy, const void *dh, const void *v, const void *gamma, const float *rstd, void *dx,
           void *dgamma, void *workspace, size_t workspace_bytes, int64_t M, int64_t N, float eps, float offset,
           int dtype, hipStream_t stream)
{
    if (!gamma) { // non-affine: no dgamma, no partials, no finalizer
        if (dgamma)
            return fail(RMSNORM_EINVAL, "dgamma given without gamma");
        int64_t programs = 0;
        return do_partials(dy, v, nullptr, rstd, dh, dx, workspace, workspace_bytes, &programs, M, N, eps, offset,
                           dtype, stream);
    }
    if (!dgamma)
        return fail(RMSNORM_EINVAL, "dgamma is null");
    if (dtype_known(dtype) && !aligned(dgamma, (size_t)elem_bytes(dtype)))
        return fail(RMSNORM_EINVAL, "dgamma not aligned to its element size");
    int64_t programs = 0;
    ColsOut cols{dgamma, nullptr, false};
    int rc = do_partials(dy, v, gamma, rstd, dh, dx, workspace, workspace_bytes, &programs, M, N, eps, offset,
                         dtype, stream, nullptr, &cols);
    if (rc || cols.done) // the one-launch backward has written dgamma
        return rc;
    return do_finalize(static_cast<const float *>(workspace), programs, N, dgamma, dtype, stream);
}

// Fixed device scratch for rmsnorm_bwd_noalloc: the partial rows (and an
// rstd recomputed when the caller has none) of one backward, for callers that
// cannot allocate.  Each device holds its own copy for the life of the
// process.  In host code the array's name is only a stand-in for the device
// symbol: the device address of each device's copy comes from
// hipGetSymbolAddress, once per device (with that device current), and only
// that address is ever passed to a kernel.  Nothing in it needs clearing: the
// backward writes every partial row and every recomputed rstd it later reads.
constexpr size_t kScratchBytes = RMSNORM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(RMSNORM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(RMSNORM_EHIP, "device %d out of range", dev);
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr)
                return fail(RMSNORM_EHIP, "device address of the scratch buffer on device %d: %s", dev,
                            hipGetErrorString(e));
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RMSNORM_OK;
}

int workspace_for(int op_a, int op_b, int64_t M, int64_t N, int dtype, size_t *bytes)
{
    if (!bytes)
        return fail(RMSNORM_EINVAL, "bytes is null");
    int rc = check_common(M, N, dtype, 0.0f, 0.0f);
    if (rc)
        return rc;
    int cus = 0;
    if ((rc = device_cus(&cus)))
        return rc;
    int64_t need = 0;
    for (int op : {op_a, op_b})
        for (bool vec_ok : {true, false}) {
            rmsnorm_plan p;
            // sized for the two-stage layout, which the stage entry point
            // runs, also where the full backward takes one launch
            if (select_plan(op, M, N, dtype, vec_ok, cus, &p) == RMSNORM_OK &&
                (p.path != RMSNORM_PATH_ROWS_COLS || two_stage(&p, M, N, dtype, cus)) && p.workspace_bytes > need)
                need = p.workspace_bytes;
        }
    *bytes = (size_t)need;
    return ok();
}

} // namespace

extern "C" {

int rmsnorm_fwd(const void *x, const void *gamma, void *y, float *rstd, int64_t M, int64_t N, float eps,
                float offset, int dtype, rmsnorm_stream_t stream)
{
    return do_fwd(x, nullptr, gamma, y, nullptr, rstd, M, N, eps, offset, dtype, stream, false);
}

int rmsnorm_fused_add_fwd(const void *x, const void *residual, const void *gamma, void *y, void *h_out,
                          float *rstd, int64_t M, int64_t N, float eps, float offset, int dtype,
                          rmsnorm_stream_t stream)
{
    return do_fwd(x, residual, gamma, y, h_out, rstd, M, N, eps, offset, dtype, stream, true);
}

int rmsnorm_fwd_fp8(const void *x, const void *gamma, void *y8, float *rstd, const float *scale, float *amax,
                    void *workspace, size_t workspace_bytes, int64_t M, int64_t N, float eps, float offset,
                    int dtype, rmsnorm_stream_t stream)
{
    const Fp8Out f8{scale, amax, workspace, workspace_bytes};
    return do_fwd(x, nullptr, gamma, y8, nullptr, rstd, M, N, eps, offset, dtype, stream, false, &f8);
}

int rmsnorm_fused_add_fwd_fp8(const void *x, const void *residual, const void *gamma, void *y8, void *h_out,
                              float *rstd, const float *scale, float *amax, void *workspace,
                              size_t workspace_bytes, int64_t M, int64_t N, float eps, float offset, int dtype,
                              rmsnorm_stream_t stream)
{
    const Fp8Out f8{scale, amax, workspace, workspace_bytes};
    return do_fwd(x, residual, gamma, y8, h_out, rstd, M, N, eps, offset, dtype, stream, true, &f8);
}

int rmsnorm_fwd_fp8_workspace_bytes(int64_t M, int64_t N, int dtype, size_t *bytes)
{
    if (!bytes)
        return fail(RMSNORM_EINVAL, "bytes is null");
    int rc = check_common(M, N, dtype, 0.0f, 0.0f);
    if (rc)
        return rc;
    int cus = 0;
    if ((rc = device_cus(&cus)))
        return rc;
    int64_t need = 0;
    for (int op : {RMSNORM_OP_FWD_FP8, RMSNORM_OP_FUSED_ADD_FWD_FP8})
        for (bool vec_ok : {true, false}) {
            rmsnorm_plan p;
            if (select_plan(op, M, N, dtype, vec_ok, cus, &p) == RMSNORM_OK && p.workspace_bytes > need)
                need = p.workspace_bytes;
        }
    *bytes = (size_t)need;
    return ok();
}

int rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, size_t *bytes)
{
    return workspace_for(RMSNORM_OP_BWD, RMSNORM_OP_FUSED_ADD_BWD, M, N, dtype, bytes);
}

int layernorm_fwd(const void *x, const void *gamma, const void *beta, void *y, float *mean, float *rstd, int64_t M,
                  int64_t N, float eps, float offset, int dtype, rmsnorm_stream_t stream)
{
    const LnFwd ln{beta, mean};
    return do_fwd(x, nullptr, gamma, y, nullptr, rstd, M, N, eps, offset, dtype, stream, false, nullptr, &ln);
}

int layernorm_fused_add_fwd(const void *x, const void *residual, const void *gamma, const void *beta, void *y,
                            void *h_out, float *mean, float *rstd, int64_t M, int64_t N, float eps, float offset,
                            int dtype, rmsnorm_stream_t stream)
{
    const LnFwd ln{beta, mean};
    return do_fwd(x, residual, gamma, y, h_out, rstd, M, N, eps, offset, dtype, stream, true, nullptr, &ln);
}

int layernorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype, size_t *bytes)
{
    return workspace_for(RMSNORM_OP_LN_BWD, RMSNORM_OP_LN_FUSED_ADD_BWD, M, N, dtype, bytes);
}

int layernorm_bwd(const void *dy, const void *x, const void *gamma, const float *mean, const float *rstd, void *dx,
                  void *dgamma, void *dbeta, void *workspace, size_t workspace_bytes, int64_t M, int64_t N,
                  float eps, float offset, int dtype, rmsnorm_stream_t stream)
{
    return do_ln_bwd(dy, nullptr, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace, workspace_bytes, M, N, eps,
                     offset, dtype, stream);
}

int layernorm_fused_add_bwd(const void *dy, const void *dh, const void *h, const void *gamma, const float *mean,
                            const float *rstd, void *dx, void *dgamma, void *dbeta, void *workspace,
                            size_t workspace_bytes, int64_t M, int64_t N, float eps, float offset, int dtype,
                            rmsnorm_stream_t stream)
{
    return do_ln_bwd(dy, dh, h, gamma, mean, rstd, dx, dgamma, dbeta, workspace, workspace_bytes, M, N, eps,
                     offset, dtype, stream);
}

int rmsnorm_bwd(const void *dy, const void *x, const void *gamma, const float *rstd, void *dx, void *dgamma,
                void *workspace, size_t workspace_bytes, int64_t M, int64_t N, float eps, float offset, int dtype,
                rmsnorm_stream_t stream)
{
    return do_bwd(dy, nullptr, x, gamma, rstd, dx, dgamma, workspace, workspace_bytes, M, N, eps, offset, dtype,
                  stream);
}

int rmsnorm_fused_add_bwd(const void *dy, const void *dh, const void *h, const void *gamma, const float *rstd,
                          void *dx, void *dgamma, void *workspace, size_t workspace_bytes, int64_t M, int64_t N,
                          float eps, float offset, int dtype, rmsnorm_stream_t stream)
{
    // With no incoming residual gradient the fused backward is the plain one on h.
    return do_bwd(dy, dh, h, gamma, rstd, dx, dgamma, workspace, workspace_bytes, M, N, eps, offset, dtype,
                  stream);
}

int rmsnorm_bwd_noalloc(const void *dy, const void *x, const void *gamma, const float *rstd, void *dx, void *dgamma,
                        int64_t M, int64_t N, float eps, float offset, int dtype, rmsnorm_stream_t stream)
{
    void *ws = nullptr;
    int rc = scratch_address(&ws);
    if (rc)
        return rc;
    rc = do_bwd(dy, nullptr, x, gamma, rstd, dx, dgamma, ws, kScratchBytes, M, N, eps, offset, dtype, stream);
    if (rc == RMSNORM_EWORKSPACE) {
        char why[sizeof g_err];
        std::snprintf(why, sizeof why, "%s", g_err);
        return fail(rc, "rmsnorm_bwd_noalloc: this call needs more than the fixed %zu-byte scratch (%s); use "
                        "rmsnorm_bwd with a workspace", kScratchBytes, why);
    }
    return rc;
}

int rmsnorm_bwd_partials(const void *dy, const void *v, const void *gamma, const float *rstd, const void *dh,
                         void *dx, void *workspace, size_t workspace_bytes, int64_t *programs, int64_t M,
                         int64_t N, float eps, float offset, int dtype, rmsnorm_stream_t stream)
{
    if (!programs)
        return fail(RMSNORM_EINVAL, "programs is null");
    return do_partials(dy, v, gamma, rstd, dh, dx, workspace, workspace_bytes, programs, M, N, eps, offset, dtype,
                       stream);
}

int rmsnorm_dgamma_finalize(const float *partials, int64_t programs, int64_t N, void *dgamma, int dtype,
                            rmsnorm_stream_t stream)
{
    return do_finalize(partials, programs, N, dgamma, dtype, stream);
}

int rmsnorm_query_plan(int op, int64_t M, int64_t N, int dtype, int vec_ok, int num_cus, rmsnorm_plan *out)
{
    if (!out)
        return fail(RMSNORM_EINVAL, "out is null");
    int cus = num_cus;
    if (cus <= 0) {
        int rc = device_cus(&cus);
        if (rc)
            return rc;
    }
    if (op < RMSNORM_OP_FWD || op > RMSNORM_OP_LN_FUSED_ADD_BWD)
        return fail(RMSNORM_EINVAL, "op %d unknown", op);
    rmsnorm_plan p;
    int rc = plan_for(op, M, N, dtype, vec_ok != 0, cus, &p);
    if (rc)
        return rc;
    *out = p;
    return ok();
}

int rmsnorm_set_plan_override(int op, const rmsnorm_plan *plan)
{
    if (op < RMSNORM_OP_FWD || op > RMSNORM_OP_LN_FUSED_ADD_BWD)
        return fail(RMSNORM_EINVAL, "op %d unknown", op);
    if (plan == nullptr) {
        g_override[op].set = false;
        return ok();
    }
    g_override[op].plan = *plan;
    g_override[op].plan.op = op;
    g_override[op].set = true;
    return ok();
}

const char *rmsnorm_status_string(int status)
{
    switch (status) {
    case RMSNORM_OK: return "ok";
    case RMSNORM_EINVAL: return "invalid argument";
    case RMSNORM_EUNSUPPORTED: return "unsupported dtype or configuration";
    case RMSNORM_EWORKSPACE: return "workspace missing or too small";
    case RMSNORM_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *rmsnorm_last_error(void) { return g_err; }

int rmsnorm_version(void) { return RMSNORM_ABI_VERSION; }

} // extern "C"
