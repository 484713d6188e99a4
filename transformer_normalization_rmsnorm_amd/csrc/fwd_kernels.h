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
//
// LayerNorm (LN; TransformerEngine PR #583 registers matching LayerNorm
// configurations): the same layouts with two reductions per row, the mean
// first and then the sum of squared deviations of the register-held row
// (two-pass, so no cancellation between E[v^2] and E[v]^2), then
// y = (v - mean) * rstd * (gamma + offset) + beta.
#pragma once

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

template <typename T, int V, int TEAM, int K, int D, bool FUSED, bool EXACT, bool F8, bool LN>
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
    C bias[LN ? K : 1]; // LayerNorm bias, or zeros
    if constexpr (LN) {
        const T *__restrict__ beta = static_cast<const T *>(a.beta);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (beta != nullptr && (EXACT || c < nchunks))
                bias[k].load_cached(beta + (int64_t)c * V);
            else
                bias[k].zero();
        }
    }

    // Every row load is issued: lanes past the row's end re-read its last
    // chunk, and only their sums and stores are masked.
    auto load = [&](Row &b, int64_t row) __attribute__((always_inline)) {
        const int64_t base = row * N;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c0 = k * tl + lane;
            const int c = EXACT ? c0 : min(c0, nchunks - 1);
            b.x[k].load(x + base + (int64_t)c * V);
            if constexpr (FUSED)
                b.r[k].load(r + base + (int64_t)c * V);
        }
    };

    __shared__ float red[2][16];
    int parity = 0;
    auto reduce = [&](float v) __attribute__((always_inline)) {
        if constexpr (TEAM == 0) {
            v = block_sum(v, red[parity], a.threads);
            parity ^= 1;
        } else {
            v = team_sum<TEAM>(v);
        }
        return v;
    };
    // Eight or more chunks per lane in the fp8 and LayerNorm forwards: gamma
    // and the row stay packed and are unpacked where they are used, instead
    // of being held unpacked across the row loop and the reduction (bf16 fp8,
    // 8 chunks: 94 instead of 162 VGPRs).  Measured on MI355X, fp8 forward
    // 4096 x 16384 bf16 37.5 against 49.1 us, 2048 x 32768 40.3 against
    // 53.1 us; LayerNorm 2048 x 32768 56.4 against 59.9 us.  The plain
    // forward at 128 threads x 8 chunks (8192 bf16) was 2-4% slower with it.
    constexpr bool kPacked = (F8 || LN) && K >= 8;
    auto proc = [&](Row &b, int64_t row) __attribute__((always_inline)) {
        const int64_t base = row * N;
        if constexpr (kPacked) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                g[k].pin();
        }
        float ss = 0.0f; // sum of squares (LayerNorm: of the deviations from the mean)
        float mu = 0.0f; // LayerNorm: the row mean
        if constexpr (!LN) {
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
            if constexpr (kPacked) {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    b.x[k].pin();
            }
        } else {
            float s1 = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int c = k * tl + lane;
                if (EXACT || c < nchunks) {
                    if constexpr (FUSED) {
                        float f[V];
#pragma unroll
                        for (int e = 0; e < V; ++e)
                            f[e] = b.x[k].get(e) + b.r[k].get(e);
                        b.x[k].set(f);
                        b.x[k].store(h + base + (int64_t)c * V);
                    }
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        s1 += b.x[k].get(e);
                }
            }
            // the row is unpacked again after each reduction, not held twice
#pragma unroll
            for (int k = 0; k < K; ++k)
                b.x[k].pin();
            mu = reduce(s1) * inv_n;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int c = k * tl + lane;
                if (EXACT || c < nchunks) {
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float t = b.x[k].get(e) - mu;
                        ss = fmaf(t, t, ss);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < K; ++k)
                b.x[k].pin();
        }
        ss = reduce(ss);
        const float rs = rsqrtf(fmaf(ss, inv_n, a.eps));
        if (rstd != nullptr)
            rstd[row] = rs; // every lane of the team stores the same value
        if constexpr (LN) {
            if (a.mean != nullptr)
                a.mean[row] = mu;
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
                float f[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    if constexpr (LN)
                        f[e] = fmaf((b.x[k].get(e) - mu) * rs, g[k].get(e) + a.offset, bias[k].get(e));
                    else
                        f[e] = (b.x[k].get(e) * rs) * (g[k].get(e) + a.offset);
                }
                store_row_out<T, V, F8>(y, base + (int64_t)c * V, f, scale, am);
            }
        }
    };

    row_pipeline<D, Row>((int64_t)blockIdx.x * tpb + team, a.grid * tpb, a.M, load, proc);
    if constexpr (F8)
        write_amax_part(am, a);
}

// Any N: pass 1 sums squares (LayerNorm: the values, then a second pass the
// squared deviations) and writes h for fused-add; the last pass writes y.
// Lane t owns the chunks t, t + nt, ...  Its first KS chunks are loaded once,
// in the first pass, and wait in LDS (each lane reads back only its own, so no
// barrier) for the later passes; chunks beyond them are read again from
// memory (from cache): x, or for fused-add the h chunk the lane itself stored
// in pass 1.  h may overwrite r, so forming x + r again would read h in place
// of r; the lane's own earlier store is what its later load of the same
// address returns.  The KS chunks are loaded unconditionally, a chunk past
// the row's end re-reading its last one, so that their loads stay in flight
// together.
template <typename T, int V, bool FUSED, bool F8, bool LN, int KS>
__global__ void __launch_bounds__(1024) fwd_loop_kernel(FwdArgs a)
{
    using C = Chunk<T, V>;
    const int nt = a.threads;
    const int N = a.N;
    const int nchunks = N / V;
    const float inv_n = 1.0f / (float)N;
    const T *__restrict__ x = static_cast<const T *>(a.x);
    const T *__restrict__ gamma = static_cast<const T *>(a.gamma);
    const T *__restrict__ beta = static_cast<const T *>(a.beta);
    const T *r = static_cast<const T *>(a.r);
    T *h = static_cast<T *>(a.h);
    void *__restrict__ y = a.y;
    const float scale = F8 ? *a.scale : 1.0f;
    float am = 0.0f;
    extern __shared__ __align__(16) unsigned char fwd_lds[]; // [KS][nt] chunks
    auto staged = [&](int j) __attribute__((always_inline)) {
        return reinterpret_cast<C *>(fwd_lds + ((size_t)j * nt + threadIdx.x) * sizeof(C));
    };

    // chunk c of the row at base: x, or round(x + r) for fused-add (pass 1)
    auto row_chunk = [&](int64_t base, int c) __attribute__((always_inline)) {
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
        return v;
    };
    // chunk c again in a later pass: x, or the h this lane stored in pass 1
    auto row_chunk_again = [&](int64_t base, int c) __attribute__((always_inline)) {
        C v;
        if constexpr (FUSED)
            v.load_cached(h + base + (int64_t)c * V);
        else
            v.load_cached(x + base + (int64_t)c * V);
        return v;
    };

    __shared__ float red[2][16];
    int parity = 0;
    for (int64_t row = blockIdx.x; row < a.M; row += a.grid) {
        const int64_t base = row * N;
        // first pass: load (write h), stage, and sum the values (LayerNorm)
        // or their squares
        float s1 = 0.0f;
        auto first = [&](const C &v) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if constexpr (LN)
                    s1 += v.get(e);
                else
                    s1 = fmaf(v.get(e), v.get(e), s1);
            }
        };
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int c = (int)threadIdx.x + j * nt;
            int cc = min(c, nchunks - 1);
            pin_vgpr(cc);
            const C v = row_chunk(base, cc);
            *staged(j) = v;
            if (c < nchunks) {
                if constexpr (FUSED)
                    v.store(h + base + (int64_t)c * V);
                first(v);
            }
        }
        for (int c = (int)threadIdx.x + KS * nt; c < nchunks; c += nt) {
            const C v = row_chunk(base, c);
            if constexpr (FUSED)
                v.store(h + base + (int64_t)c * V);
            first(v);
        }
        s1 = block_sum(s1, red[parity], a.threads);
        parity ^= 1;
        float mu = 0.0f, ss = s1;
        if constexpr (LN) { // second pass: squared deviations from the mean
            mu = s1 * inv_n;
            float s2 = 0.0f;
            auto dev2 = [&](const C &v) __attribute__((always_inline)) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float t = v.get(e) - mu;
                    s2 = fmaf(t, t, s2);
                }
            };
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                if ((int)threadIdx.x + j * nt < nchunks)
                    dev2(*staged(j));
            }
            for (int c = (int)threadIdx.x + KS * nt; c < nchunks; c += nt)
                dev2(row_chunk_again(base, c));
            ss = block_sum(s2, red[parity], a.threads);
            parity ^= 1;
        }
        const float rs = rsqrtf(fmaf(ss, inv_n, a.eps));
        if (threadIdx.x == 0) {
            if (a.rstd != nullptr)
                a.rstd[row] = rs;
            if constexpr (LN) {
                if (a.mean != nullptr)
                    a.mean[row] = mu;
            }
        }
        if (y == nullptr)
            continue;
        auto out = [&](const C &v, int c) __attribute__((always_inline)) {
            float w[V], bb[V];
            if (gamma != nullptr) {
                C g;
                g.load_cached(gamma + (int64_t)c * V);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    w[e] = g.get(e) + a.offset;
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    w[e] = 1.0f;
            }
            if (LN && beta != nullptr) {
                C bc;
                bc.load_cached(beta + (int64_t)c * V);
#pragma unroll
                for (int e = 0; e < V; ++e)
                    bb[e] = bc.get(e);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    bb[e] = 0.0f;
            }
            float f[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if constexpr (LN)
                    f[e] = fmaf((v.get(e) - mu) * rs, w[e], bb[e]);
                else
                    f[e] = (v.get(e) * rs) * w[e];
            }
            store_row_out<T, V, F8>(y, base + (int64_t)c * V, f, scale, am);
        };
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            const int c = (int)threadIdx.x + j * nt;
            if (c < nchunks)
                out(*staged(j), c);
        }
        for (int c = (int)threadIdx.x + KS * nt; c < nchunks; c += nt)
            out(row_chunk_again(base, c), c);
    }
    if constexpr (F8)
        write_amax_part(am, a);
}

template <typename T, int V, int TEAM, int K, int D, bool FUSED, bool F8, bool LN>
static void launch_fwd_rows(const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
    const int lanes = TEAM ? TEAM : p.threads;
    if constexpr (V > 1) {
        if ((int64_t)lanes * K == a.N / V) {
            hipLaunchKernelGGL((fwd_rows_kernel<T, V, TEAM, K, D, FUSED, true, F8, LN>), grid, block, 0, s, a);
            return;
        }
    }
    hipLaunchKernelGGL((fwd_rows_kernel<T, V, TEAM, K, D, FUSED, false, F8, LN>), grid, block, 0, s, a);
}

template <typename T, bool FUSED, bool F8, bool LN>
static hipError_t dispatch_fwd(const rmsnorm_plan &p, FwdArgs a, hipStream_t s)
{
    constexpr int VV = 16 / (int)sizeof(T);
    a.threads = p.threads;
    a.grid = p.grid;
    if (p.path == RMSNORM_PATH_LOOP || a.y == nullptr) {
        // statistics-only forwards (y == nullptr) also take the looped kernel,
        // one 256-thread workgroup per row, the grid capped below 2^31
        // work-items (the kernel strides over the rows)
        a.threads = p.path == RMSNORM_PATH_LOOP ? p.threads : 256;
        a.grid = p.path == RMSNORM_PATH_LOOP ? p.grid : std::min<int64_t>(a.M, (kMaxWorkItems - 1) / 256);
        const dim3 g2((unsigned)a.grid), b2((unsigned)a.threads);
        // 16-byte chunks: up to eight per lane staged in LDS (four when the
        // row has at most four per lane).  Per-element rows are not staged,
        // nor the fp8 output: with a third of the bytes to write it kept more
        // workgroups per CU without the LDS (measured on MI355X, 2048 x 40960
        // bf16: 62.6 us unstaged against 74.2 us staged; RMSNorm 72.4 -> 68.0
        // us, LayerNorm 88.3 -> 79.6 us with staging)
        const int64_t per_lane = ((int64_t)a.N / p.vec + a.threads - 1) / a.threads;
        const size_t slot = (size_t)a.threads * 16;
        if (p.vec == VV) {
            if constexpr (F8) {
                hipLaunchKernelGGL((fwd_loop_kernel<T, VV, FUSED, F8, LN, 0>), g2, b2, 0, s, a);
            } else {
                if (per_lane <= 4)
                    hipLaunchKernelGGL((fwd_loop_kernel<T, VV, FUSED, F8, LN, 4>), g2, b2, 4 * slot, s, a);
                else
                    hipLaunchKernelGGL((fwd_loop_kernel<T, VV, FUSED, F8, LN, 8>), g2, b2, 8 * slot, s, a);
            }
        } else {
            hipLaunchKernelGGL((fwd_loop_kernel<T, 1, FUSED, F8, LN, 0>), g2, b2, 0, s, a);
        }
        return hipGetLastError();
    }
    const bool vec = (p.vec == VV);
    // fp8 output and LayerNorm exist for the layouts without prefetch, and
    // LayerNorm (which also holds beta) for at most kLnFwdMaxChunks chunks
#define RMSNORM_CASE(VEC, TEAM, K, D)                                                        \
    if constexpr ((!F8 && !LN) || (D == 0 && (!LN || K <= kLnFwdMaxChunks))) {               \
        if (vec == (VEC == 1) && p.team == TEAM && p.chunks == K && p.depth == D) {          \
            launch_fwd_rows<T, (VEC == 1 ? VV : 1), TEAM, K, D, FUSED, F8, LN>(p, a, s);     \
            return hipGetLastError();                                                        \
        }                                                                                    \
    }
    RMSNORM_FWD_ROWS_CONFIGS(RMSNORM_CASE)
#undef RMSNORM_CASE
    return hipErrorInvalidConfiguration;
}

template <typename T, bool FUSED>
static hipError_t dispatch_fwd_kind(FwdKind kind, const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s)
{
    switch (kind) {
    case FWD_RMS_FP8: return dispatch_fwd<T, FUSED, true, false>(p, a, s);
    case FWD_LN: return dispatch_fwd<T, FUSED, false, true>(p, a, s);
    default: return dispatch_fwd<T, FUSED, false, false>(p, a, s);
    }
}

// Forward launch for storage type T; explicitly instantiated once per type in
// fwd_<type>.hip, so that the three types compile in parallel.
template <typename T>
hipError_t launch_fwd_typed(bool fused, FwdKind kind, const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s)
{
    return fused ? dispatch_fwd_kind<T, true>(kind, p, a, s) : dispatch_fwd_kind<T, false>(kind, p, a, s);
}

} // namespace rmsnorm
