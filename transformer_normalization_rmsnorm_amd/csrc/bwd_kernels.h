// RMSNorm backward kernels for gfx950 (plain and fused residual add).
//
// With w = gamma + offset, g = dy * w, xhat = v * rstd and
// c = (1/N) sum_j g_j xhat_j, a row's input gradient is
//     dx = rstd * (g - xhat * c)  [+ dh for the fused-add op],
// evaluated here as dx = rstd * g - v * (rstd^3 * dot / N) with
// dot = sum_j g_j v_j, and dgamma_j = sum over rows of dy_j * xhat_j.
//
// Structure (FlyDSL PR #855, "Hybrid atomic / two-stage backward" and
// "512-thread vec8 fast path"): a bounded persistent grid of P workgroups walks
// the rows in a grid-stride loop, loads w once per workgroup, keeps each row's
// v and dy in VGPRs across both passes, writes dx with 16-byte stores and
// accumulates float32 dgamma partials in registers; at the end each workgroup
// writes one partial row.  A finalizer then sums the [P, N] partials in a
// fixed order and writes dgamma in the parameter dtype: no atomics, no clear
// and no separate conversion kernel.  Unlike the page's kernel, each team keeps
// D further rows in flight (row_pipeline) while it reduces and writes the
// current one, so HBM latency overlaps the work instead of stalling it.  With
// 16 to 31 rows per program and one chunk per lane, two rows share each
// workgroup reduction (the kDepthPairs instance, plan rows_per_step = 2).
//
// Rows wider than one chunk per lane of a 1024-lane workgroup (8192 bf16 /
// 4096 fp32 elements; the page's scope stops at N = 8192 and keeps atomics
// above) use the same kernel with w_regs = 0: gamma is re-read through the
// cache with every row instead of held as fp32 w, and the row's packed
// registers are pinned between the two passes, so that up to 32 bf16 (16
// fp32) elements per lane and 1024 lanes -- rows of 32768 bf16 / 16384 fp32
// elements -- stay resident without spilling.
//
// LayerNorm (LN; TransformerEngine PR #583 registers matching LayerNorm
// configurations) runs on the same layouts: with xhat = (v - mean) * rstd and
// g = dy * w, one paired reduction gives mean(g) and mean(g * xhat), then
// dx = rstd * (g - mean(g) - xhat * mean(g * xhat)) [+ dh]; each program keeps
// two accumulator sets, dgamma (dy * xhat) and dbeta (dy), and writes two
// partial rows, which the finalizer folds with a second row of workgroups.
//
// With few rows per program one launch does both (the COLS instances, plan
// path RMSNORM_PATH_ROWS_COLS): dgamma_j needs no row sum, so workgroups after
// the row programs each read dy and x over all rows for a slab of columns
// and write dgamma (and dbeta) directly, in a fixed order.  The row programs
// then write no partial rows, and load their rows through the cache, where
// that second read finds them.
#pragma once

#include "device_common.h"
#include "rmsnorm_internal.h"

namespace rmsnorm {

template <typename T, int V, int K, bool WR, bool FUSED>
struct BwdRow {
    Chunk<T, V> v[K];
    Chunk<T, V> dy[K];
    Chunk<T, V> g[WR ? 1 : K]; // gamma, when it travels with the row
    Chunk<T, V> dh[FUSED ? K : 1];
    float rs;
    float mu; // LayerNorm: the row mean
};

// One-launch backward for few rows (RMSNORM_PATH_ROWS_COLS): the workgroups
// after the row programs sum dgamma_j = sum_i dy_ij * v_ij * rstd_i directly,
// by columns, instead of the row programs writing partial rows for a second
// kernel.  dgamma needs no row sum, so the two roles are independent and run
// side by side; the column workgroups read dy and v a second time (2MN
// elements), which at these sizes costs less than the dependent launch it
// saves.  Column workgroup b owns col_cs consecutive 16-byte chunks of the
// row; its thread t takes the rows t / col_cs, t / col_cs + threads / col_cs,
// ..., four at a time with their loads in flight together.  The per-thread
// sums are folded by lane exchange within each wave and then in wave order
// through LDS, so the order depends only on M, the workgroup size and col_cs.
// LayerNorm (LN): dgamma_j = sum_i dy_ij * (v_ij - mean_i) * rstd_i and
// dbeta_j = sum_i dy_ij, the same way.
// The loads go through the cache: a 128-byte line holds 8 / col_cs slabs,
// and the workgroups that share it are given one XCD (the dispatcher sends
// workgroup g to XCD g mod 8, so b, b + 8, b + 16, ... get consecutive slabs).
template <typename T, int V, bool LN>
__device__ __forceinline__ void dgamma_columns(const BwdArgs &a)
{
    using C = Chunk<T, V>;
    const int cs = a.col_cs;
    const int nt = a.threads;
    const int N = a.N;
    const int nchunks = N / V;
    const int64_t b = (int64_t)blockIdx.x - a.grid;
    const int64_t ncol = (nchunks + cs - 1) / cs;
    const int64_t per = (ncol + 7) / 8;
    const int64_t slab = (b % 8) * per + b / 8;
    if (slab >= ncol) // one of the workgroups that round the launch up to whole XCD rounds
        return;
    const int lc = (int)threadIdx.x % cs;
    const int phase = (int)threadIdx.x / cs;
    const int nphase = nt / cs;
    const int c = (int)(slab * cs) + lc;
    const T *__restrict__ dyp = static_cast<const T *>(a.dy);
    const T *__restrict__ vp = static_cast<const T *>(a.v);
    constexpr int S = LN ? 2 : 1; // sums per element: dgamma (and dbeta)
    float acc[S][V];
#pragma unroll
    for (int q = 0; q < S; ++q) {
#pragma unroll
        for (int e = 0; e < V; ++e)
            acc[q][e] = 0.0f;
    }
    auto add = [&](const C &d, const C &x, float rs, float mu) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            if constexpr (LN) {
                acc[0][e] = fmaf(d.get(e), (x.get(e) - mu) * rs, acc[0][e]);
                acc[1][e] += d.get(e);
            } else {
                acc[0][e] = fmaf(d.get(e), x.get(e) * rs, acc[0][e]);
            }
        }
    };
    if (c < nchunks) {
        int64_t r = phase;
        for (; r + 3 * (int64_t)nphase < a.M; r += 4 * (int64_t)nphase) {
            C d[4], x[4];
            float rs[4], mu[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t rr = r + u * (int64_t)nphase;
                d[u].load_cached(dyp + rr * N + (int64_t)c * V);
                x[u].load_cached(vp + rr * N + (int64_t)c * V);
                rs[u] = a.rstd[rr];
                mu[u] = LN ? a.mean[rr] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                add(d[u], x[u], rs[u], mu[u]);
        }
        for (; r < a.M; r += nphase) {
            C d, x;
            d.load_cached(dyp + r * N + (int64_t)c * V);
            x.load_cached(vp + r * N + (int64_t)c * V);
            add(d, x, a.rstd[r], LN ? a.mean[r] : 0.0f);
        }
    }
    // lanes l and l ^ cs, l ^ 2 cs, ... of a wave hold the same chunk
    for (int off = cs; off < 64; off <<= 1) {
#pragma unroll
        for (int q = 0; q < S; ++q) {
#pragma unroll
            for (int e = 0; e < V; ++e)
                acc[q][e] += __shfl_xor(acc[q][e], off);
        }
    }
    // [wave][sum][chunk in slab * V + element]: cs * V <= 64
    __shared__ float colred[16][S][64];
    const int w = (int)threadIdx.x >> 6, l = (int)threadIdx.x & 63;
    if (l < cs) {
#pragma unroll
        for (int q = 0; q < S; ++q) {
#pragma unroll
            for (int e = 0; e < V; ++e)
                colred[w][q][l * V + e] = acc[q][e];
        }
    }
    __syncthreads();
    const int j = (int)threadIdx.x % 64; // element j of the slab, sum q
    const int q = (int)threadIdx.x / 64;
    if (j < cs * V && q < S) {
        float s = colred[0][q][j];
        for (int wv = 1; wv < nt / 64; ++wv)
            s += colred[wv][q][j];
        const int64_t col = slab * cs * V + j;
        T *out = static_cast<T *>(q == 0 ? a.dgamma : a.dbeta);
        if (col < N && out != nullptr)
            out[col] = to_storage<T>(s);
    }
}

// COLS: the one-launch backward (col_cs > 0): the row programs, then from
// `grid` on the dgamma (and dbeta) column workgroups.  They read dy and x a
// second time, so its row programs load the rows through the cache, where
// the second read finds them (the two-stage backward streams them with the
// nontemporal hint).
template <typename T, int V, int TEAM, int K, int D, bool WR, int BOUND, bool FUSED, bool EXACT, bool LN, bool COLS>
__global__ void __launch_bounds__(BOUND) bwd_rows_kernel(BwdArgs a)
{
    if constexpr (COLS) {
        static_assert(bwd_cols_layout(TEAM, K, WR, V), "column workgroups run beside the layouts bwd_cols_layout names");
        if (blockIdx.x >= a.grid) {
            dgamma_columns<T, V, LN>(a);
            return;
        }
    }
    using Row = BwdRow<T, V, K, WR, FUSED>;
    const int tl = TEAM ? TEAM : a.threads;
    const int lane = TEAM ? (int)(threadIdx.x & (TEAM - 1)) : (int)threadIdx.x;
    const int tpb = TEAM ? a.threads / TEAM : 1;
    const int team = TEAM ? (int)(threadIdx.x / TEAM) : 0;
    const int N = a.N;
    const int nchunks = N / V;
    const float inv_n = 1.0f / (float)N;
    const T *__restrict__ dyp = static_cast<const T *>(a.dy);
    const T *__restrict__ vp = static_cast<const T *>(a.v);
    const T *__restrict__ gp = static_cast<const T *>(a.gamma);
    const T *dhp = static_cast<const T *>(a.dh); // dx may alias dh
    T *dxp = static_cast<T *>(a.dx);
    const float *__restrict__ rstd = a.rstd;

    // Wide LayerNorm rows (bwd_dbeta_in_lds) keep the dbeta accumulators in
    // LDS instead of registers: each lane owns the slots of its own columns
    // (no barriers), laid out as float4 planes [V / 4][nchunks] so that a
    // wavefront's 16-byte accesses are contiguous.
    constexpr bool BL = bwd_dbeta_in_lds(LN, FUSED, TEAM, K, V);
    constexpr int KW = WR ? K : 1;
    constexpr int KB = (LN && !BL) ? K : 1;
    constexpr int NPL = V / 4 > 0 ? V / 4 : 1; // float4 planes of the LDS dbeta row
    float w[KW][V], acc[K][V]; // w = gamma + offset, or 1 for the non-affine op
    float accb[KB][V];         // LayerNorm: the dbeta accumulators (in registers)
    extern __shared__ float4 lds_db[]; // [NPL][nchunks] when BL
    // (COLS: the column workgroups sum dgamma and dbeta; the row programs
    // accumulate nothing)
    if constexpr (BL && !COLS) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
#pragma unroll
                for (int h = 0; h < NPL; ++h)
                    lds_db[h * nchunks + c] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
#pragma unroll
        for (int e = 0; e < V; ++e)
            acc[k][e] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
#pragma unroll
        for (int e = 0; e < V; ++e)
            accb[k][e] = 0.0f;
    }
    if constexpr (WR) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            Chunk<T, V> g;
            if (gp != nullptr && (EXACT || c < nchunks))
                g.load_cached(gp + (int64_t)c * V);
#pragma unroll
            for (int e = 0; e < V; ++e)
                w[k][e] = (EXACT || c < nchunks) ? (gp != nullptr ? g.get(e) + a.offset : 1.0f) : 0.0f;
        }
    }
    // Every load is unconditional (see row_pipeline): lanes past the row's end
    // re-read its last chunk and only their stores are masked; without gamma
    // the row's weight loads read dy's first row and the values are ignored.
    const T *__restrict__ gsrc = gp != nullptr ? gp : dyp;
    const bool affine = gp != nullptr;
    // weight of element e of chunk k of row buffer b
    auto weight = [&](const Row &b, int k, int e) __attribute__((always_inline)) {
        if constexpr (WR)
            return w[k][e];
        else
            return affine ? b.g[k].get(e) + a.offset : 1.0f;
    };

    auto load = [&](Row &b, int64_t row) __attribute__((always_inline)) {
        const int64_t base = row * N;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c0 = k * tl + lane;
            int c = EXACT ? c0 : min(c0, nchunks - 1);
            // LayerNorm: form the chunk addresses per row rather than hold the
            // row-invariant ones (gamma's) in registers across the loop
            if constexpr (LN)
                pin_vgpr(c);
            if constexpr (COLS) {
                b.v[k].load_cached(vp + base + (int64_t)c * V);
                b.dy[k].load_cached(dyp + base + (int64_t)c * V);
            } else {
                b.v[k].load(vp + base + (int64_t)c * V);
                b.dy[k].load(dyp + base + (int64_t)c * V);
            }
            if constexpr (!WR)
                b.g[k].load_cached(gsrc + (int64_t)c * V);
            if constexpr (FUSED)
                b.dh[k].load(dhp + base + (int64_t)c * V);
        }
        b.rs = rstd[row];
        if constexpr (LN)
            b.mu = a.mean[row];
    };

    __shared__ float red[2][LN ? 64 : 32]; // floats a slot: block_sum 16, block_sum2 32, block_sum4 64
    int parity = 0;
    // values unpacked in the first pass are formed again in the second where
    // registers are scarce (see below)
    auto pin_row = [&](Row &b) __attribute__((always_inline)) {
        if constexpr (!WR || TEAM != 0) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                b.v[k].pin();
                b.dy[k].pin();
                if constexpr (!WR)
                    b.g[k].pin();
                if constexpr (FUSED)
                    b.dh[k].pin();
            }
        }
    };
    // element e of a row chunk: get_unfused where it measured faster for
    // binary16 (RMSNorm, workgroup teams with w in registers, one vector chunk
    // per lane and at most one row in flight: 4096 x 4096 21.7 -> 20.3 us);
    // with two rows in flight (16384 x 2048: 44.6 -> 46.4 us) and for
    // LayerNorm (4096 x 4096: 24.9 -> 25.5 us) the extra registers cost more
    auto elem = [&](const Chunk<T, V> &c, int e) __attribute__((always_inline)) {
        if constexpr (!LN && TEAM == 0 && WR && K == 1 && D <= 1 && V > 1)
            return c.get_unfused(e);
        else
            return c.get(e);
    };
    auto proc_ln = [&](Row &b, int64_t row) __attribute__((always_inline)) {
        const float rs = b.rs, mu = b.mu;
        float sg = 0.0f, sgx = 0.0f; // sum g, sum g * xhat
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float gg = elem(b.dy[k], e) * weight(b, k, e);
                    sg += gg;
                    sgx = fmaf(gg, (elem(b.v[k], e) - mu) * rs, sgx);
                }
            }
        }
        pin_row(b);
        if constexpr (TEAM == 0) {
            block_sum2(sg, sgx, red[parity], a.threads);
            parity ^= 1;
        } else {
            sg = team_sum<TEAM>(sg);
            sgx = team_sum<TEAM>(sgx);
        }
        const float c1 = sg * inv_n, c2 = sgx * inv_n;
        const int64_t base = row * N;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = elem(b.dy[k], e);
                    const float xh = (elem(b.v[k], e) - mu) * rs;
                    float dxv = rs * fmaf(-xh, c2, d * weight(b, k, e) - c1);
                    if constexpr (FUSED)
                        dxv += b.dh[k].get(e);
                    o[e] = dxv;
                    if constexpr (!COLS)
                        acc[k][e] = fmaf(d, xh, acc[k][e]);
                    if constexpr (LN && !BL && !COLS)
                        accb[k][e] += d;
                }
                if constexpr (BL && !COLS) {
#pragma unroll
                    for (int h = 0; h < NPL; ++h) {
                        float4 t = lds_db[h * nchunks + c];
                        t.x += b.dy[k].get(4 * h + 0);
                        t.y += b.dy[k].get(4 * h + 1);
                        t.z += b.dy[k].get(4 * h + 2);
                        t.w += b.dy[k].get(4 * h + 3);
                        lds_db[h * nchunks + c] = t;
                    }
                    // keep each chunk's LDS update in place: hoisting every
                    // chunk's read to the top of the pass costs 8 VGPRs a chunk
                    asm volatile("" ::: "memory");
                }
                Chunk<T, V> out;
                out.set(o);
                out.store(dxp + base + (int64_t)c * V);
            }
        }
    };
    auto proc = [&](Row &b, int64_t row) __attribute__((always_inline)) {
        if constexpr (LN) {
            proc_ln(b, row);
            return;
        }
        float dot = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    dot = fmaf(elem(b.dy[k], e) * weight(b, k, e), elem(b.v[k], e), dot);
            }
        }
        // Values unpacked for the dot are formed again in the second pass where
        // registers are scarce: gamma-per-row layouts and sub-workgroup teams
        // (measured on MI355X: 262144 x 128 bf16 3% faster).  Workgroup teams
        // with w in registers have registers to spare at one program per CU,
        // and keeping the unpacked row there is 1.5% faster (4096 x 4096,
        // 16384 x 8192 bf16).
        pin_row(b);
        if constexpr (TEAM == 0) {
            dot = block_sum(dot, red[parity], a.threads);
            parity ^= 1;
        } else {
            dot = team_sum<TEAM>(dot);
        }
        const float rs = b.rs;
        const float kc = rs * rs * rs * dot * inv_n; // dx = rs * g - v * kc
        const int64_t base = row * N;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float xv = elem(b.v[k], e);
                    const float d = elem(b.dy[k], e);
                    float dxv = fmaf(rs, d * weight(b, k, e), -xv * kc);
                    if constexpr (FUSED)
                        dxv += b.dh[k].get(e);
                    o[e] = dxv;
                    if constexpr (!COLS)
                        acc[k][e] = fmaf(d, xv * rs, acc[k][e]);
                }
                Chunk<T, V> out;
                out.set(o);
                out.store(dxp + base + (int64_t)c * V);
            }
        }
    };

    if constexpr (D == kDepthPairs) {
        static_assert(bwd_pairs_compiled(LN, FUSED, TEAM, K, 1, WR, V), "two rows per step: not this layout");
        // Two rows per step (rows_per_step = 2): both rows' dots go through
        // one workgroup reduction (block_sum2, one barrier), and the next
        // two rows are loaded before the current two are worked on.  A
        // program's rows r0, r0 + s, r0 + 2s, ... pair up in order; a
        // missing second row (odd count) is loaded clamped to the last row
        // and neither written nor accumulated.
        // LayerNorm: the two rows' mean(g) and mean(g * xhat) go through one
        // four-sum reduction.
        auto proc2_ln = [&](Row &b0, Row &b1, int64_t row, bool second) __attribute__((always_inline)) {
            float sg0 = 0.0f, sgx0 = 0.0f, sg1 = 0.0f, sgx1 = 0.0f;
            const int c = lane; // one chunk per lane
            if (EXACT || c < nchunks) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float g0 = elem(b0.dy[0], e) * weight(b0, 0, e);
                    const float g1 = elem(b1.dy[0], e) * weight(b1, 0, e);
                    sg0 += g0;
                    sg1 += g1;
                    sgx0 = fmaf(g0, (elem(b0.v[0], e) - b0.mu) * b0.rs, sgx0);
                    sgx1 = fmaf(g1, (elem(b1.v[0], e) - b1.mu) * b1.rs, sgx1);
                }
            }
            block_sum4(sg0, sgx0, sg1, sgx1, red[parity], a.threads);
            parity ^= 1;
            auto pass2 = [&](Row &b, float sg, float sgx, int64_t r) __attribute__((always_inline)) {
                const float rs = b.rs, mu = b.mu;
                const float c1 = sg * inv_n, c2 = sgx * inv_n;
                if (EXACT || c < nchunks) {
                    float o[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float d = elem(b.dy[0], e);
                        const float xh = (elem(b.v[0], e) - mu) * rs;
                        o[e] = rs * fmaf(-xh, c2, d * weight(b, 0, e) - c1);
                        if constexpr (!COLS) {
                            acc[0][e] = fmaf(d, xh, acc[0][e]);
                            accb[0][e] += d;
                        }
                    }
                    Chunk<T, V> out;
                    out.set(o);
                    out.store(dxp + r * N + (int64_t)c * V);
                }
            };
            pass2(b0, sg0, sgx0, row);
            if (second)
                pass2(b1, sg1, sgx1, row + a.grid);
        };
        auto proc2 = [&](Row &b0, Row &b1, int64_t row, bool second) __attribute__((always_inline)) {
            if constexpr (LN) {
                proc2_ln(b0, b1, row, second);
                return;
            }
            float dot0 = 0.0f, dot1 = 0.0f;
            const int c = lane; // one chunk per lane
            if (EXACT || c < nchunks) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    dot0 = fmaf(elem(b0.dy[0], e) * weight(b0, 0, e), elem(b0.v[0], e), dot0);
                    dot1 = fmaf(elem(b1.dy[0], e) * weight(b1, 0, e), elem(b1.v[0], e), dot1);
                }
            }
            block_sum2(dot0, dot1, red[parity], a.threads);
            parity ^= 1;
            auto pass2 = [&](Row &b, float dot, int64_t r) __attribute__((always_inline)) {
                const float rs = b.rs;
                const float kc = rs * rs * rs * dot * inv_n; // dx = rs * g - v * kc
                if (EXACT || c < nchunks) {
                    float o[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float xv = elem(b.v[0], e);
                        const float d = elem(b.dy[0], e);
                        o[e] = fmaf(rs, d * weight(b, 0, e), -xv * kc);
                        if constexpr (FUSED)
                            o[e] += b.dh[0].get(e);
                        if constexpr (!COLS)
                            acc[0][e] = fmaf(d, xv * rs, acc[0][e]);
                    }
                    Chunk<T, V> out;
                    out.set(o);
                    out.store(dxp + r * N + (int64_t)c * V);
                }
            };
            pass2(b0, dot0, row);
            if (second)
                pass2(b1, dot1, row + a.grid);
        };
        const int64_t stride = a.grid, M = a.M, row0 = blockIdx.x;
        const int64_t last = row0 < M ? row0 + (M - 1 - row0) / stride * stride : M - 1;
        auto clamp = [&](int64_t r) __attribute__((always_inline)) { return r < last ? r : last; };
        Row buf[2][2];
        load(buf[0][0], clamp(row0));
        load(buf[0][1], clamp(row0 + stride));
        for (int64_t base = row0; base < M; base += 4 * stride) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int64_t r = base + (int64_t)s * 2 * stride;
                if (r >= M)
                    break;
                load(buf[s ^ 1][0], clamp(r + 2 * stride));
                load(buf[s ^ 1][1], clamp(r + 3 * stride));
                proc2(buf[s][0], buf[s][1], r, r + stride < M);
            }
        }
    } else {
        row_pipeline<D, Row>((int64_t)blockIdx.x * tpb + team, a.grid * tpb, a.M, load, proc);
    }

    if constexpr (COLS)
        return; // the column workgroups write dgamma and dbeta
    if (a.partials == nullptr) // no dgamma (non-affine) and no dbeta
        return;
    float *__restrict__ part = a.partials + (int64_t)blockIdx.x * a.ld;
    float *__restrict__ partb = a.partials + (a.grid + (int64_t)blockIdx.x) * a.ld; // LayerNorm dbeta
    if constexpr (TEAM == 0) {
        // LayerNorm rows of one or two chunks per lane, and RMSNorm rows of
        // two, write their partial rows with the nontemporal hint, as the
        // finalizer reads them (measured on MI355X with one workspace reused
        // call after call, LayerNorm backward of 1024 x 8192 bf16: 23.4 ->
        // 21.0 us; within noise with a fresh workspace per call).  RMSNorm
        // rows of one chunk write them cached: with the hint (set in buffer
        // stores) the backward of 4096 x 4096 and 1024 x 8192 bf16 took 1.4%
        // and 4.9% longer.  Wider rows keep cached stores: there the hint
        // cost 2048 x 32768 bf16 3.7 us.
        constexpr bool kNtPartials = K == 2 || (K == 1 && LN);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
                if constexpr (kNtPartials)
                    store_f32_nt<V>(part + (int64_t)c * V, acc[k]);
                else
                    store_f32<V>(part + (int64_t)c * V, acc[k]);
                if constexpr (BL) {
#pragma unroll
                    for (int h = 0; h < NPL; ++h)
                        *reinterpret_cast<float4 *>(partb + (int64_t)c * V + 4 * h) = lds_db[h * nchunks + c];
                } else if constexpr (LN && K <= 2) {
                    store_f32_nt<V>(partb + (int64_t)c * V, accb[k]);
                } else if constexpr (LN) {
                    store_f32<V>(partb + (int64_t)c * V, accb[k]);
                }
            }
        }
    } else {
        // Several teams per workgroup: add their partials in team order.
        extern __shared__ float team_acc[]; // [sets][tpb][N]
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int c = k * tl + lane;
            if (EXACT || c < nchunks) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    team_acc[team * N + c * V + e] = acc[k][e];
                    if constexpr (LN)
                        team_acc[(tpb + team) * N + c * V + e] = accb[k][e];
                }
            }
        }
        __syncthreads();
        for (int j = threadIdx.x; j < N; j += a.threads) {
            float s = team_acc[j];
            for (int t = 1; t < tpb; ++t)
                s += team_acc[t * N + j];
            part[j] = s;
            if constexpr (LN) {
                float sb = team_acc[tpb * N + j];
                for (int t = 1; t < tpb; ++t)
                    sb += team_acc[(tpb + t) * N + j];
                partb[j] = sb;
            }
        }
    }
}

// Any N: per row, pass 1 forms the row sums (dot; LayerNorm: mean(g) and
// mean(g * xhat)), pass 2 re-reads the row (from cache) and writes dx.  Lane
// t owns the chunks t, t + nt, t + 2 nt, ...  The v chunks of its first KA
// chunks (16-byte ones) wait in LDS between the passes, so pass 2 re-reads
// only dy and gamma for them (1024 x 65536 bf16: 141.4 -> 132.4 us; 1024 x
// 32768 fp32: 123.7 -> 107.0 us).  The dgamma (and dbeta)
// accumulators of its first KA chunks stay in registers for all the
// workgroup's rows and are written once at the end; those of later chunks
// (rows wider than KA x nt x V) are read, updated and written back in the
// partial rows with every row (the lane owns them, so the read-modify-write
// is private).  The KA chunks are loaded unconditionally, a chunk past the
// row's end re-reading its last one, so that their loads stay in flight
// together (a load that may be skipped makes the compiler wait for all
// outstanding ones).
template <typename T, int V, bool FUSED, bool LN, int KA>
__global__ void __launch_bounds__(1024) bwd_loop_kernel(BwdArgs a)
{
    using C = Chunk<T, V>;
    const int nt = a.threads;
    const int N = a.N;
    const int nchunks = N / V;
    const float inv_n = 1.0f / (float)N;
    const T *__restrict__ dyp = static_cast<const T *>(a.dy);
    const T *__restrict__ vp = static_cast<const T *>(a.v);
    const T *__restrict__ gp = static_cast<const T *>(a.gamma);
    const T *dhp = static_cast<const T *>(a.dh);
    T *dxp = static_cast<T *>(a.dx);
    // without gamma the weight loads read dy's first row and are ignored
    const T *__restrict__ gsrc = gp != nullptr ? gp : dyp;
    // null: no dgamma (non-affine) and no dbeta
    float *part = a.partials ? a.partials + (int64_t)blockIdx.x * a.ld : nullptr;
    float *partb = (LN && a.partials) ? a.partials + (a.grid + (int64_t)blockIdx.x) * a.ld : nullptr;
    auto wgt = [&](const C &g, int e) __attribute__((always_inline)) {
        return gp != nullptr ? g.get(e) + a.offset : 1.0f;
    };
    float acc[KA][V], accb[LN ? KA : 1][V];
    // v of the register slots, kept between the passes: [KA][nt] chunks, each
    // lane reading back only its own (no barrier); vector chunks only
    extern __shared__ __align__(16) unsigned char loop_lds[];
    auto staged = [&](int j) __attribute__((always_inline)) {
        return reinterpret_cast<C *>(loop_lds + ((size_t)j * nt + threadIdx.x) * sizeof(C));
    };
#pragma unroll
    for (int j = 0; j < KA; ++j) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            acc[j][e] = 0.0f;
            if constexpr (LN)
                accb[j][e] = 0.0f;
        }
    }

    __shared__ float red[2][32];
    int parity = 0;
    for (int64_t row = blockIdx.x; row < a.M; row += a.grid) {
        const bool first = (row == (int64_t)blockIdx.x);
        const int64_t base = row * N;
        const float rs = a.rstd[row];
        const float mu = LN ? a.mean[row] : 0.0f;
        float s1 = 0.0f, s2 = 0.0f; // RMSNorm: s1 = dot; LayerNorm: sum g, sum g * xhat
        auto sums = [&](const C &v, const C &d, const C &g) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float gg = d.get(e) * wgt(g, e);
                if constexpr (LN) {
                    s1 += gg;
                    s2 = fmaf(gg, (v.get(e) - mu) * rs, s2);
                } else {
                    s1 = fmaf(gg, v.get(e), s1);
                }
            }
        };
#pragma unroll
        for (int j = 0; j < KA; ++j) {
            const int c = (int)threadIdx.x + j * nt;
            int cc = min(c, nchunks - 1);
            pin_vgpr(cc); // form the addresses per row rather than hold them
            C v, d, g;
            v.load_cached(vp + base + (int64_t)cc * V);
            d.load_cached(dyp + base + (int64_t)cc * V);
            g.load_cached(gsrc + (int64_t)cc * V);
            if constexpr (V > 1)
                *staged(j) = v;
            if (c < nchunks)
                sums(v, d, g);
            // two chunks in flight at a time: the accumulators take the
            // registers that hoisting every chunk's loads would need
            if (j % 2 == 1)
                asm volatile("" ::: "memory");
        }
        for (int c = (int)threadIdx.x + KA * nt; c < nchunks; c += nt) {
            C v, d, g;
            v.load_cached(vp + base + (int64_t)c * V);
            d.load_cached(dyp + base + (int64_t)c * V);
            g.load_cached(gsrc + (int64_t)c * V);
            sums(v, d, g);
        }
        if constexpr (LN) {
            block_sum2(s1, s2, red[parity], a.threads);
        } else {
            s1 = block_sum(s1, red[parity], a.threads);
        }
        parity ^= 1;
        const float kc = rs * rs * rs * s1 * inv_n;       // RMSNorm
        const float c1 = s1 * inv_n, c2 = s2 * inv_n;     // LayerNorm
        // dx of one chunk, with its dgamma / dbeta contributions added to pa / pb
        auto chunk_dx = [&](int c, const C &v, const C &d, const C &g, const C &dh, float (&pa)[V],
                            float (&pb)[V]) __attribute__((always_inline)) {
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float dv = d.get(e);
                float dxv;
                if constexpr (LN) {
                    const float xh = (v.get(e) - mu) * rs;
                    dxv = rs * fmaf(-xh, c2, dv * wgt(g, e) - c1);
                    pa[e] = fmaf(dv, xh, pa[e]);
                    pb[e] += dv;
                } else {
                    const float xv = v.get(e);
                    dxv = fmaf(rs, dv * wgt(g, e), -xv * kc);
                    pa[e] = fmaf(dv, xv * rs, pa[e]);
                }
                if constexpr (FUSED)
                    dxv += dh.get(e);
                o[e] = dxv;
            }
            C out;
            out.set(o);
            out.store(dxp + base + (int64_t)c * V);
        };
#pragma unroll
        for (int j = 0; j < KA; ++j) {
            const int c = (int)threadIdx.x + j * nt;
            int cc = min(c, nchunks - 1);
            pin_vgpr(cc);
            C v, d, g, dh;
            if constexpr (V > 1)
                v = *staged(j);
            else
                v.load_cached(vp + base + (int64_t)cc * V);
            d.load_cached(dyp + base + (int64_t)cc * V);
            g.load_cached(gsrc + (int64_t)cc * V);
            if constexpr (FUSED)
                dh.load_cached(dhp + base + (int64_t)cc * V);
            if (c < nchunks)
                chunk_dx(c, v, d, g, dh, acc[j], accb[LN ? j : 0]);
            if (j % 2 == 1)
                asm volatile("" ::: "memory");
        }
        for (int c = (int)threadIdx.x + KA * nt; c < nchunks; c += nt) {
            C v, d, g, dh;
            v.load_cached(vp + base + (int64_t)c * V);
            d.load_cached(dyp + base + (int64_t)c * V);
            g.load_cached(gsrc + (int64_t)c * V);
            if constexpr (FUSED)
                dh.load_cached(dhp + base + (int64_t)c * V);
            float pa[V], pb[V];
            if (first || part == nullptr) {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    pa[e] = pb[e] = 0.0f;
            } else {
                load_f32<V>(part + (int64_t)c * V, pa);
                if constexpr (LN)
                    load_f32<V>(partb + (int64_t)c * V, pb);
            }
            chunk_dx(c, v, d, g, dh, pa, pb);
            if (part != nullptr) {
                store_f32<V>(part + (int64_t)c * V, pa);
                if constexpr (LN)
                    store_f32<V>(partb + (int64_t)c * V, pb);
            }
        }
    }
    if (part == nullptr)
        return;
#pragma unroll
    for (int j = 0; j < KA; ++j) {
        const int c = (int)threadIdx.x + j * nt;
        if (c < nchunks) {
            store_f32<V>(part + (int64_t)c * V, acc[j]);
            if constexpr (LN)
                store_f32<V>(partb + (int64_t)c * V, accb[j]);
        }
    }
}

// dgamma_j = round_T(sum_p partials[p, j]).  Workgroup b owns the 32 columns
// [32b, 32b + 32) (one 128-byte line per partial row): lane (cg, pg) sums
// float4 column group cg over the rows p = pg, pg + 32, pg + 64, ... in
// increasing p, issuing kFinDepth loads before adding them so that their
// latencies overlap.  The 32 group sums are then folded in a fixed tree: the
// 8 groups that share a wave by lane exchange (xor 8, 16, 32), the 4 wave
// sums through LDS in wave order.  The order depends only on P, so dgamma is
// bit-reproducible.
template <typename T>
__global__ void __launch_bounds__(kFinThreads) finalize_kernel(const float *__restrict__ part0, int64_t P,
                                                               int64_t ld, int64_t N, T *__restrict__ dg0,
                                                               T *__restrict__ db)
{
    // workgroup row 0: dgamma from the first P partial rows; row 1
    // (LayerNorm): dbeta from the next P
    const float *__restrict__ part = part0 + (int64_t)blockIdx.y * P * ld;
    T *__restrict__ dg = blockIdx.y ? db : dg0;
    if (dg == nullptr)
        return; // the whole workgroup: this output was not asked for
    constexpr int CG = kFinColsPerBlock / 4; // float4 groups per workgroup
    constexpr int PG = kFinThreads / CG;     // partial-row groups
    constexpr int kFinDepth = 8;
    static_assert(kFinThreads % 64 == 0 && 64 % CG == 0, "a wave holds whole row groups");
    const int cg = threadIdx.x % CG;
    const int pg = threadIdx.x / CG;
    const int64_t col = (int64_t)blockIdx.x * kFinColsPerBlock + cg * 4;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (col < ld) {
        for (int64_t p0 = pg; p0 < P; p0 += (int64_t)PG * kFinDepth) {
            float4 t[kFinDepth];
#pragma unroll
            for (int i = 0; i < kFinDepth; ++i) {
                const int64_t p = p0 + (int64_t)i * PG;
                f32x4_t u = {0.0f, 0.0f, 0.0f, 0.0f};
                if (p < P) // read once: nontemporal, like the rows
                    u = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(part + p * ld + col));
                t[i] = make_float4(u.x, u.y, u.z, u.w);
            }
#pragma unroll
            for (int i = 0; i < kFinDepth; ++i) {
                s.x += t[i].x;
                s.y += t[i].y;
                s.z += t[i].z;
                s.w += t[i].w;
            }
        }
    }
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
        s.x += __shfl_xor(s.x, off);
        s.y += __shfl_xor(s.y, off);
        s.z += __shfl_xor(s.z, off);
        s.w += __shfl_xor(s.w, off);
    }
    constexpr int NW = kFinThreads / 64;
    __shared__ float4 red[NW][CG];
    if (threadIdx.x % 64 < CG)
        red[threadIdx.x / 64][cg] = s;
    __syncthreads();
    if (pg == 0) {
        float4 t = red[0][cg];
#pragma unroll
        for (int i = 1; i < NW; ++i) {
            const float4 u = red[i][cg];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        const float f[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (col + e < N) {
                dg[col + e] = to_storage<T>(f[e]);
            }
        }
    }
}

template <typename T, int V, int TEAM, int K, int D, bool WR, int BOUND, bool FUSED, bool LN>
static hipError_t launch_bwd_rows(const rmsnorm_plan &p, const BwdArgs &a, hipStream_t s)
{
    // the one-launch backward adds its dgamma column workgroups after the row programs
    const int64_t cols = a.col_cs > 0 ? bwd_col_workgroups(a.N / V, a.col_cs) : 0;
    const dim3 grid((unsigned)(p.grid + cols)), block((unsigned)p.threads);
    const int lanes = TEAM ? TEAM : p.threads;
    const size_t sets = LN ? 2 : 1;
    // sub-workgroup teams: their partial rows; LayerNorm with dbeta in LDS:
    // the dbeta row (N floats)
    constexpr bool BL = bwd_dbeta_in_lds(LN, FUSED, TEAM, K, V);
    const size_t lds = TEAM ? sets * (size_t)(p.threads / TEAM) * (size_t)a.N * sizeof(float)
                            : (BL ? (size_t)a.N * sizeof(float) : 0);
    constexpr int kTiling = bwd_tiling(LN, FUSED, (int)sizeof(T), V, TEAM, K, BOUND);
    const bool exact = (int64_t)lanes * K == a.N / V;
    if (cols) {
        // (layouts of one chunk per lane have both instances)
        if constexpr (bwd_cols_layout(TEAM, K, WR, V) && kTiling == TILING_ANY) {
            if (exact)
                hipLaunchKernelGGL((bwd_rows_kernel<T, V, TEAM, K, D, WR, BOUND, FUSED, true, LN, true>), grid, block,
                                   lds, s, a);
            else
                hipLaunchKernelGGL((bwd_rows_kernel<T, V, TEAM, K, D, WR, BOUND, FUSED, false, LN, true>), grid, block,
                                   lds, s, a);
            return hipGetLastError();
        } else {
            return hipErrorInvalidConfiguration; // the selector plans column workgroups only on these layouts
        }
    }
    if constexpr (V > 1 && kTiling != TILING_MASKED_ONLY) {
        if (exact) {
            hipLaunchKernelGGL((bwd_rows_kernel<T, V, TEAM, K, D, WR, BOUND, FUSED, true, LN, false>), grid, block, lds, s,
                               a);
            return hipGetLastError();
        }
    }
    if constexpr (kTiling == TILING_EXACT_ONLY) {
        return hipErrorInvalidConfiguration; // ragged row: the selector never plans it
    } else {
        hipLaunchKernelGGL((bwd_rows_kernel<T, V, TEAM, K, D, WR, BOUND, FUSED, false, LN, false>), grid, block, lds, s,
                           a);
        return hipGetLastError();
    }
}

// Register accumulator slots of the looped backward (chunks per lane whose
// dgamma / dbeta sums stay in registers): the most that compile for 1024
// threads (128 VGPRs) without spilling.  bf16 chunks unpack to twice the
// registers they load into, so they get fewer; LayerNorm holds two sets.
// (bf16 RMSNorm fits seven slots when v is re-read from memory, six with v
// staged in LDS, and six staged are faster at 40960 and slower at 65536.)
template <typename T, int V, bool LN>
constexpr int loop_slots()
{
    if constexpr (V > 1 && sizeof(T) == 2)
        return LN ? 3 : 6;
    else
        return LN ? 4 : 8;
}

template <typename T, bool FUSED, bool LN>
static hipError_t dispatch_bwd(const rmsnorm_plan &p, BwdArgs a, hipStream_t s)
{
    constexpr int VV = 16 / (int)sizeof(T);
    a.threads = p.threads;
    a.grid = p.grid;
    const dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
    if (p.path == RMSNORM_PATH_LOOP) {
        // register accumulator slots: four for rows of at most four chunks per
        // lane, else the most that fit 1024-thread workgroups without spilling
        constexpr int KV = loop_slots<T, VV, LN>(), K1 = loop_slots<T, 1, LN>();
        constexpr int KV4 = KV < 4 ? KV : 4, K14 = K1 < 4 ? K1 : 4;
        const int64_t per_lane = ((int64_t)a.N / p.vec + p.threads - 1) / p.threads;
        const bool few = per_lane <= 4;
        const size_t bv = (size_t)p.threads * 16, b1 = 0; // LDS per slot (vector chunks only)
        if (p.vec == VV) {
            if (few)
                hipLaunchKernelGGL((bwd_loop_kernel<T, VV, FUSED, LN, KV4>), grid, block, KV4 * bv, s, a);
            else
                hipLaunchKernelGGL((bwd_loop_kernel<T, VV, FUSED, LN, KV>), grid, block, KV * bv, s, a);
        } else {
            if (few)
                hipLaunchKernelGGL((bwd_loop_kernel<T, 1, FUSED, LN, K14>), grid, block, K14 * b1, s, a);
            else
                hipLaunchKernelGGL((bwd_loop_kernel<T, 1, FUSED, LN, K1>), grid, block, K1 * b1, s, a);
        }
        return hipGetLastError();
    }
    const bool vec = (p.vec == VV);
    if constexpr (bwd_pairs_compiled(LN, FUSED, 0, 1, 1, true, VV)) {
        if (p.rows_per_step == 2) { // complete_plan admits it only for bwd_pairs_compiled layouts
            if (!(vec && p.team == 0 && p.chunks == 1 && p.depth == 1 && p.w_regs == 1 &&
                  p.threads <= bwd_pairs_bound(FUSED, LN)))
                return hipErrorInvalidConfiguration;
            return launch_bwd_rows<T, VV, 0, 1, kDepthPairs, true, bwd_pairs_bound(FUSED, LN), FUSED, LN>(p, a, s);
        }
    }
#define RMSNORM_CASE(VEC, TEAM, K, D, WR, BOUND, FBOUND)                                      \
    if constexpr ((FUSED ? FBOUND : BOUND) > 0) {                                                 \
        if (vec == (VEC == 1) && p.team == TEAM && p.chunks == K && p.depth == D && p.w_regs == WR) { \
            return launch_bwd_rows<T, (VEC == 1 ? VV : 1), TEAM, K, D, WR == 1, (FUSED ? FBOUND : BOUND), FUSED, \
                                   LN>(p, a, s);                                                  \
        }                                                                                         \
    }
    if constexpr (LN) {
        RMSNORM_LN_BWD_ROWS_CONFIGS(RMSNORM_CASE)
    } else {
        RMSNORM_BWD_ROWS_CONFIGS(RMSNORM_CASE)
    }
#undef RMSNORM_CASE
    return hipErrorInvalidConfiguration;
}

// Backward and finalizer launches for storage type T; explicitly instantiated
// once per type in bwd_<type>.hip.
template <typename T>
hipError_t launch_bwd_typed(bool fused, bool ln, const rmsnorm_plan &p, const BwdArgs &a, hipStream_t s)
{
    if (ln)
        return fused ? dispatch_bwd<T, true, true>(p, a, s) : dispatch_bwd<T, false, true>(p, a, s);
    return fused ? dispatch_bwd<T, true, false>(p, a, s) : dispatch_bwd<T, false, false>(p, a, s);
}

template <typename T>
hipError_t launch_finalize_typed(const float *partials, int64_t programs, int64_t ld, int64_t N, void *dgamma,
                                 void *dbeta, hipStream_t s)
{
    const dim3 grid((unsigned)((ld + kFinColsPerBlock - 1) / kFinColsPerBlock), dbeta ? 2u : 1u),
        block(kFinThreads);
    hipLaunchKernelGGL((finalize_kernel<T>), grid, block, 0, s, partials, programs, ld, N, static_cast<T *>(dgamma),
                       static_cast<T *>(dbeta));
    return hipGetLastError();
}

} // namespace rmsnorm
