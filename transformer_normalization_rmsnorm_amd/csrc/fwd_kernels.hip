// RMSNorm forward kernels for gfx950 (plain and fused residual add).
//
// Per row: rstd = 1/sqrt(mean(v^2) + eps), y = round_T(v * rstd * (gamma +
// offset)); fused-add first forms h = round_T(x + r) and normalises the stored
// h.  All arithmetic is float32 with one rounding of each stored output
// (Liger-Kernel PR #1388, Summary and "Results" llama mode; FlyDSL PR #855
// "Implementation": two-pass row math with a block reduction; fused-add as a
// compile-time specialization).
//
// ROWS path: a team of lanes owns one row at a time and keeps it in VGPRs
// between the sum of squares and the scaling, so x (and r) are read from HBM
// once.  A team is 8..64 lanes of one wavefront (reduction by DPP/ds_swizzle
// only) or the whole workgroup (wavefront sums, then one LDS exchange).
// LOOP path: any N and any alignment; the row is re-read in the second pass.
#include <algorithm>

#include "device_common.h"
#include "rmsnorm_internal.h"

namespace rmsnorm {

template <typename T, int V, int K, bool FUSED>
struct FwdRow {
    Chunk<T, V> x[K];
    Chunk<T, V> r[FUSED ? K : 1];
};

// Forward on the ROWS path (y required).  gamma is loaded once per team,
// together with the first rows; each team then runs the row pipeline (D rows
// in flight).  With a grid covering every row each team handles one row; a
// smaller grid makes the kernel persistent.  EXACT: lanes x chunks covers the
// row exactly, so no lane is masked.
template <typename T, int V, int TEAM, int K, int D, bool FUSED, bool EXACT>
__global__ void __launch_bounds__(fwd_rows_bound_rule(TEAM, K)) fwd_rows_kernel(FwdArgs a)
{
    using C = Chunk<T, V>;
    using Row = FwdRow<T, V, K, FUSED>;
    const int tl = TEAM ? TEAM : a.threads; // lanes per row
    const int lane = TEAM ? (int)(threadIdx.x & (TEAM - 1)) : (int)threadIdx.x;
    const int tpb = TEAM ? a.threads / TEAM : 1; // teams per workgroup
    const int team = TEAM ? (int)(threadIdx.x / TEAM) : 0;
    const int N = a.N;
    const int nchunks = N / V;
    const float inv_n = 1.0f / (float)N;
    const T *__restrict__ x = static_cast<const T *>(a.x);
    const T *__restrict__ gamma = static_cast<const T *>(a.gamma);
    const T *r = static_cast<const T *>(a.r); // h may alias r
    T *h = static_cast<T *>(a.h);
    T *__restrict__ y = static_cast<T *>(a.y);
    float *__restrict__ rstd = a.rstd;

    C g[K]; // gamma, or ones for the non-affine op (offset is then 0)
    if (gamma != nullptr) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks)
                g[k].load_cached(gamma + (int64_t)c * V);
        }
    } else {
        float one[V];
#pragma unroll
        for (int e = 0; e < V; ++e)
            one[e] = 1.0f;
#pragma unroll
        for (int k = 0; k < K; ++k)
            g[k].set(one);
    }

    auto load = [&](Row &b, int64_t row) __attribute__((always_inline)) {
        const int64_t base = row * N;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
                b.x[k].load(x + base + (int64_t)c * V);
                if constexpr (FUSED)
                    b.r[k].load(r + base + (int64_t)c * V);
            }
        }
    };

    __shared__ float red[2][16];
    int parity = 0;
    auto proc = [&](Row &b, int64_t row) __attribute__((always_inline)) {
        const int64_t base = row * N;
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
                if constexpr (FUSED) {
                    float f[V];
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        f[e] = b.x[k].get(e) + b.r[k].get(e);
                    b.x[k].set(f); // h, rounded to the storage type
                    b.x[k].store(h + base + (int64_t)c * V);
                }
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float t = b.x[k].get(e);
                    ss = fmaf(t, t, ss);
                }
            }
        }
        if constexpr (TEAM == 0) {
            ss = block_sum(ss, red[parity], a.threads);
            parity ^= 1;
        } else {
            ss = team_sum<TEAM>(ss);
        }
        const float rs = rsqrtf(fmaf(ss, inv_n, a.eps));
        if (rstd != nullptr)
            rstd[row] = rs; // every lane of the team stores the same value
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
                float f[V];
#pragma unroll
                for (int e = 0; e < V; ++e)
                    f[e] = (b.x[k].get(e) * rs) * (g[k].get(e) + a.offset);
                C o;
                o.set(f);
                o.store(y + base + (int64_t)c * V);
            }
        }
    };

    row_pipeline<D, Row>((int64_t)blockIdx.x * tpb + team, a.grid * tpb, a.M, load, proc);
}

// Any N: pass 1 sums squares (and writes h for fused-add), pass 2 re-reads the
// row (recomputing h from x and r) and writes y.
template <typename T, int V, bool FUSED>
__global__ void __launch_bounds__(1024) fwd_loop_kernel(FwdArgs a)
{
    using C = Chunk<T, V>;
    const int nt = a.threads;
    const int N = a.N;
    const int nchunks = N / V;
    const float inv_n = 1.0f / (float)N;
    const T *__restrict__ x = static_cast<const T *>(a.x);
    const T *__restrict__ gamma = static_cast<const T *>(a.gamma);
    const T *r = static_cast<const T *>(a.r);
    T *h = static_cast<T *>(a.h);
    T *__restrict__ y = static_cast<T *>(a.y);

    __shared__ float red[2][16];
    int parity = 0;
    for (int64_t row = blockIdx.x; row < a.M; row += a.grid) {
        const int64_t base = row * N;
        float ss = 0.0f;
        for (int c = threadIdx.x; c < nchunks; c += nt) {
            C v;
            v.load_cached(x + base + (int64_t)c * V);
            if constexpr (FUSED) {
                C rc;
                rc.load_cached(r + base + (int64_t)c * V);
                float f[V];
#pragma unroll
                for (int e = 0; e < V; ++e)
                    f[e] = v.get(e) + rc.get(e);
                v.set(f);
                v.store(h + base + (int64_t)c * V);
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float t = v.get(e);
                ss = fmaf(t, t, ss);
            }
        }
        ss = block_sum(ss, red[parity], a.threads);
        parity ^= 1;
        const float rs = rsqrtf(fmaf(ss, inv_n, a.eps));
        if (a.rstd != nullptr && threadIdx.x == 0)
            a.rstd[row] = rs;
        if (y == nullptr)
            continue;
        for (int c = threadIdx.x; c < nchunks; c += nt) {
            C v;
            v.load_cached(x + base + (int64_t)c * V);
            if constexpr (FUSED) {
                C rc;
                rc.load_cached(r + base + (int64_t)c * V);
                float f[V];
#pragma unroll
                for (int e = 0; e < V; ++e)
                    f[e] = v.get(e) + rc.get(e);
                v.set(f);
            }
            float f[V];
            if (gamma != nullptr) {
                C g;
                g.load_cached(gamma + (int64_t)c * V);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    f[e] = (v.get(e) * rs) * (g.get(e) + a.offset);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    f[e] = v.get(e) * rs;
            }
            C o;
            o.set(f);
            o.store(y + base + (int64_t)c * V);
        }
    }
}

template <typename T, int V, int TEAM, int K, int D, bool FUSED>
static void launch_fwd_rows(const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
    const int lanes = TEAM ? TEAM : p.threads;
    if constexpr (V > 1) {
        if ((int64_t)lanes * K == a.N / V) {
            hipLaunchKernelGGL((fwd_rows_kernel<T, V, TEAM, K, D, FUSED, true>), grid, block, 0, s, a);
            return;
        }
    }
    hipLaunchKernelGGL((fwd_rows_kernel<T, V, TEAM, K, D, FUSED, false>), grid, block, 0, s, a);
}

template <typename T, bool FUSED>
static hipError_t dispatch_fwd(const rmsnorm_plan &p, FwdArgs a, hipStream_t s)
{
    constexpr int VV = 16 / (int)sizeof(T);
    a.threads = p.threads;
    a.grid = p.grid;
    if (p.path == RMSNORM_PATH_LOOP || a.y == nullptr) {
        // rstd-only forwards (y == nullptr) also take the looped kernel
        const dim3 grid((unsigned)std::min<int64_t>(a.M, 1 << 30)), block(256);
        a.threads = p.path == RMSNORM_PATH_LOOP ? p.threads : 256;
        a.grid = p.path == RMSNORM_PATH_LOOP ? p.grid : grid.x;
        const dim3 g2((unsigned)a.grid), b2((unsigned)a.threads);
        if (p.vec == VV)
            hipLaunchKernelGGL((fwd_loop_kernel<T, VV, FUSED>), g2, b2, 0, s, a);
        else
            hipLaunchKernelGGL((fwd_loop_kernel<T, 1, FUSED>), g2, b2, 0, s, a);
        return hipGetLastError();
    }
    const bool vec = (p.vec == VV);
#define RMSNORM_CASE(VEC, TEAM, K, D)                                                        \
    if (vec == (VEC == 1) && p.team == TEAM && p.chunks == K && p.depth == D) {              \
        launch_fwd_rows<T, (VEC == 1 ? VV : 1), TEAM, K, D, FUSED>(p, a, s);                 \
        return hipGetLastError();                                                            \
    }
    RMSNORM_FWD_ROWS_CONFIGS(RMSNORM_CASE)
#undef RMSNORM_CASE
    return hipErrorInvalidConfiguration;
}

hipError_t launch_fwd(int dtype, bool fused, const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s)
{
    if (dtype == RMSNORM_BF16)
        return fused ? dispatch_fwd<bf16_t, true>(p, a, s) : dispatch_fwd<bf16_t, false>(p, a, s);
    return fused ? dispatch_fwd<float, true>(p, a, s) : dispatch_fwd<float, false>(p, a, s);
}

} // namespace rmsnorm
