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
//
// fp8 output (F8; TransformerEngine PR #583: the normalization output type
// may be float8 E4M3): y is written as OCP E4M3 codes of y * scale (one byte
// per element, store_e4m3), and each workgroup writes the maximum |y| it saw
// to amax_part[blockIdx.x]; amax_finalize_kernel folds those into the
// caller's amax.  One atomic max per workgroup on a single address was
// measured on MI355X at about 8.5 ns each, serialised (4096 workgroups: +35 us
// on a 21 us kernel), hence the two stages.
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
// Row output: V values rounded to T, or E4M3 codes (F8) at byte offset elem.
template <typename T, int V, bool F8>
__device__ __forceinline__ void store_row_out(void *y, int64_t elem, const float (&f)[V], float scale, float &am)
{
    if constexpr (F8) {
        store_e4m3<V>(static_cast<uint8_t *>(y) + elem, f, scale, am);
    } else {
        Chunk<T, V> o;
        o.set(f);
        o.store(static_cast<T *>(y) + elem);
    }
}

// The workgroup's maximum |y| into amax_part[blockIdx.x] (fp8 output).
__device__ __forceinline__ void write_amax_part(float am, const FwdArgs &a)
{
    __shared__ float slot[16];
    if (a.amax_part == nullptr)
        return;
    am = block_max(am, slot, a.threads);
    if (threadIdx.x == 0)
        a.amax_part[blockIdx.x] = am;
}

template <typename T, int V, int TEAM, int K, int D, bool FUSED, bool EXACT, bool F8>
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
    void *__restrict__ y = a.y;
    float *__restrict__ rstd = a.rstd;
    const float scale = F8 ? *a.scale : 1.0f;
    float am = 0.0f; // max |y| of this lane (fp8 output)

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
                store_row_out<T, V, F8>(y, base + (int64_t)c * V, f, scale, am);
            }
        }
    };

    row_pipeline<D, Row>((int64_t)blockIdx.x * tpb + team, a.grid * tpb, a.M, load, proc);
    if constexpr (F8)
        write_amax_part(am, a);
}

// Any N: pass 1 sums squares (and writes h for fused-add), pass 2 re-reads the
// row (recomputing h from x and r) and writes y.
template <typename T, int V, bool FUSED, bool F8>
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
    void *__restrict__ y = a.y;
    const float scale = F8 ? *a.scale : 1.0f;
    float am = 0.0f;

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
            store_row_out<T, V, F8>(y, base + (int64_t)c * V, f, scale, am);
        }
    }
    if constexpr (F8)
        write_amax_part(am, a);
}

// *amax = max(*amax, max_p part[p]), one workgroup.  The partials are read as
// float4 with kAmaxLoads independent loads per lane in flight, so a round
// covers kAmaxThreads * kAmaxLoads * 4 partials for one memory latency (a
// dependent loop of scalar loads cost one latency per 256 partials: about 20
// us at 16384 workgroups).  Every load is issued: lanes past the end re-read
// the last group and their values are ignored.
constexpr int kAmaxLoads = 4;

__global__ void __launch_bounds__(kAmaxThreads) amax_finalize_kernel(const float *__restrict__ part, int64_t P,
                                                                     float *amax)
{
    __shared__ float slot[16];
    float m = 0.0f;
    const int64_t P4 = P / 4;
    const float4 *__restrict__ p4 = reinterpret_cast<const float4 *>(part);
    for (int64_t b = 0; b < P4; b += (int64_t)kAmaxThreads * kAmaxLoads) {
        float4 v[kAmaxLoads];
#pragma unroll
        for (int u = 0; u < kAmaxLoads; ++u) {
            const int64_t i = b + (int64_t)u * kAmaxThreads + threadIdx.x;
            v[u] = p4[i < P4 ? i : P4 - 1];
        }
#pragma unroll
        for (int u = 0; u < kAmaxLoads; ++u) {
            const int64_t i = b + (int64_t)u * kAmaxThreads + threadIdx.x;
            if (i < P4)
                m = fmaxf(m, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
        }
    }
    for (int64_t i = P4 * 4 + threadIdx.x; i < P; i += kAmaxThreads)
        m = fmaxf(m, part[i]);
    m = block_max(m, slot, kAmaxThreads);
    if (threadIdx.x == 0)
        *amax = fmaxf(*amax, m);
}

template <typename T, int V, int TEAM, int K, int D, bool FUSED, bool F8>
static void launch_fwd_rows(const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
    const int lanes = TEAM ? TEAM : p.threads;
    if constexpr (V > 1) {
        if ((int64_t)lanes * K == a.N / V) {
            hipLaunchKernelGGL((fwd_rows_kernel<T, V, TEAM, K, D, FUSED, true, F8>), grid, block, 0, s, a);
            return;
        }
    }
    hipLaunchKernelGGL((fwd_rows_kernel<T, V, TEAM, K, D, FUSED, false, F8>), grid, block, 0, s, a);
}

template <typename T, bool FUSED, bool F8>
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
            hipLaunchKernelGGL((fwd_loop_kernel<T, VV, FUSED, F8>), g2, b2, 0, s, a);
        else
            hipLaunchKernelGGL((fwd_loop_kernel<T, 1, FUSED, F8>), g2, b2, 0, s, a);
        return hipGetLastError();
    }
    const bool vec = (p.vec == VV);
#define RMSNORM_CASE(VEC, TEAM, K, D)                                                        \
    if constexpr (!F8 || D == 0) {                                                           \
        if (vec == (VEC == 1) && p.team == TEAM && p.chunks == K && p.depth == D) {          \
            launch_fwd_rows<T, (VEC == 1 ? VV : 1), TEAM, K, D, FUSED, F8>(p, a, s);         \
            return hipGetLastError();                                                        \
        }                                                                                    \
    }
    RMSNORM_FWD_ROWS_CONFIGS(RMSNORM_CASE)
#undef RMSNORM_CASE
    return hipErrorInvalidConfiguration;
}

hipError_t launch_fwd(int dtype, bool fused, bool fp8, const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s)
{
    if (dtype == RMSNORM_BF16) {
        if (fp8)
            return fused ? dispatch_fwd<bf16_t, true, true>(p, a, s) : dispatch_fwd<bf16_t, false, true>(p, a, s);
        return fused ? dispatch_fwd<bf16_t, true, false>(p, a, s) : dispatch_fwd<bf16_t, false, false>(p, a, s);
    }
    if (fp8)
        return fused ? dispatch_fwd<float, true, true>(p, a, s) : dispatch_fwd<float, false, true>(p, a, s);
    return fused ? dispatch_fwd<float, true, false>(p, a, s) : dispatch_fwd<float, false, false>(p, a, s);
}

hipError_t launch_amax_finalize(const float *part, int64_t programs, float *amax, hipStream_t s)
{
    hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kAmaxThreads), 0, s, part, programs, amax);
    return hipGetLastError();
}

} // namespace rmsnorm
