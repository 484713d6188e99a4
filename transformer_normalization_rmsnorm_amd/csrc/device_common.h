// Device helpers for the gfx950 RMSNorm kernels: vector chunks of a row,
// bf16 / binary16 <-> f32 conversion, and wavefront / workgroup sum reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rmsnorm {

// bf16 is carried as its raw 16-bit pattern.
using bf16_t = uint16_t;

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 -> f32 is exact: the bf16 bits are the high half of the f32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two f32 -> packed bf16x2, round to nearest even, with gfx950's
// v_cvt_pk_bf16_f32 (the hardware conversion FlyDSL PR #855 uses on gfx95,
// "512-thread vec8 fast path").  Element 0 lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16(float f)
{
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// IEEE binary16 is carried as its raw 16-bit pattern too, in a type of its own
// so that the kernel templates tell it apart from bf16.
struct alignas(2) f16_t {
    uint16_t bits;
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// binary16 -> f32 is exact (v_cvt_f32_f16); f32 -> binary16 rounds to nearest
// even, with subnormal results and overflow to infinity, as the IEEE
// conversion does.  Element 0 is in the low half.
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w).x; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w).y; }
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// The two 16-bit storage types: two values per 32-bit word.
template <typename T>
struct Pair16;

template <>
struct Pair16<bf16_t> {
    static __device__ __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
    static __device__ __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
};

template <>
struct Pair16<f16_t> {
    static __device__ __forceinline__ float lo(uint32_t w) { return f16_lo(w); }
    static __device__ __forceinline__ float hi(uint32_t w) { return f16_hi(w); }
    static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
};

// One f32 value rounded to the storage type T.
template <typename T>
__device__ __forceinline__ T to_storage(float f)
{
    if constexpr (sizeof(T) == 4)
        return f;
    else
        return __builtin_bit_cast(T, (uint16_t)(Pair16<T>::pack(f, 0.0f) & 0xffffu));
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Register barrier: an empty asm statement that claims to modify `x`, so the
// compiler cannot carry values derived from `x` across it and must derive them
// again from the (packed) register afterwards.  Used between a row's two
// passes: without it the compiler keeps the unpacked fp32 copies of a bf16 row
// (and products such as dy * w) live across the reduction, which doubles the
// registers a row needs.
template <typename U>
__device__ __forceinline__ void pin_vgpr(U &x)
{
    static_assert(sizeof(U) == 4, "one 32-bit register");
    asm volatile("" : "+v"(x));
}

// A chunk is the V consecutive elements of a row that one lane moves with one
// memory instruction: 16 bytes (bf16 or binary16 x8, f32 x4) on the vector path, one
// element on the scalar path.  load/store stream the row tensors with the
// nontemporal hint (each element is touched once per call; measured on
// MI355X: about 10% more bandwidth for three-stream traffic); load_cached is
// for gamma, which every team re-reads.  pin() applies the register barrier
// to the chunk's registers.
template <typename T, int V>
struct Chunk;

// 8 elements of a 16-bit type (bf16 or binary16) in four packed words.
template <typename T>
struct Chunk16x8 {
    uint32_t w[4];
    __device__ __forceinline__ void load(const T *p)
    {
        const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    }
    __device__ __forceinline__ void load_cached(const T *p)
    {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    }
    __device__ __forceinline__ void store(T *p) const
    {
        const u32x4_t u = {w[0], w[1], w[2], w[3]};
        __builtin_nontemporal_store(u, reinterpret_cast<u32x4_t *>(p));
    }
    __device__ __forceinline__ float get(int e) const
    {
        return (e & 1) ? Pair16<T>::hi(w[e >> 1]) : Pair16<T>::lo(w[e >> 1]);
    }
    // get() for binary16 as a float the compiler may not fold back into the
    // arithmetic: hipcc otherwise turns conversions feeding an fma into
    // v_fma_mix_f32, which measured slower in the 4096 x 4096 backward (21.7
    // against 20.3 us); it costs registers, so only some layouts use it.
    // bf16 is unchanged.
    __device__ __forceinline__ float get_unfused(int e) const
    {
        float f = get(e);
        if constexpr (!std::is_same<T, bf16_t>::value)
            asm volatile("" : "+v"(f));
        return f;
    }
    __device__ __forceinline__ void set(const float (&f)[8])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = Pair16<T>::pack(f[2 * i], f[2 * i + 1]);
    }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = 0u;
    }
    __device__ __forceinline__ void pin()
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pin_vgpr(w[i]);
    }
};

// One element of a 16-bit type.
template <typename T>
struct Chunk16x1 {
    uint16_t b;
    __device__ __forceinline__ void load(const T *p)
    {
        b = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
    }
    __device__ __forceinline__ void load_cached(const T *p) { b = *reinterpret_cast<const uint16_t *>(p); }
    __device__ __forceinline__ void store(T *p) const
    {
        __builtin_nontemporal_store(b, reinterpret_cast<uint16_t *>(p));
    }
    __device__ __forceinline__ float get(int) const { return Pair16<T>::lo((uint32_t)b); }
    __device__ __forceinline__ void set(const float (&f)[1]) { b = (uint16_t)(Pair16<T>::pack(f[0], 0.0f) & 0xffffu); }
    __device__ __forceinline__ void zero() { b = 0; }
    __device__ __forceinline__ void pin()
    {
        uint32_t t = b;
        pin_vgpr(t);
        b = (uint16_t)t;
    }
};

template <>
struct Chunk<bf16_t, 8> : Chunk16x8<bf16_t> {};
template <>
struct Chunk<f16_t, 8> : Chunk16x8<f16_t> {};
template <>
struct Chunk<bf16_t, 1> : Chunk16x1<bf16_t> {};
template <>
struct Chunk<f16_t, 1> : Chunk16x1<f16_t> {};

template <>
struct Chunk<float, 4> {
    float v[4];
    __device__ __forceinline__ void load(const float *p)
    {
        const f32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    }
    __device__ __forceinline__ void load_cached(const float *p)
    {
        const float4 u = *reinterpret_cast<const float4 *>(p);
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    }
    __device__ __forceinline__ void store(float *p) const
    {
        const f32x4_t u = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(u, reinterpret_cast<f32x4_t *>(p));
    }
    __device__ __forceinline__ float get(int e) const { return v[e]; }
    __device__ __forceinline__ float get_unfused(int e) const { return v[e]; }
    __device__ __forceinline__ void set(const float (&f)[4])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = f[i];
    }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = 0.0f;
    }
    __device__ __forceinline__ void pin()
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pin_vgpr(v[i]);
    }
};

template <>
struct Chunk<float, 1> {
    float v;
    __device__ __forceinline__ void load(const float *p) { v = __builtin_nontemporal_load(p); }
    __device__ __forceinline__ void load_cached(const float *p) { v = *p; }
    __device__ __forceinline__ void store(float *p) const { __builtin_nontemporal_store(v, p); }
    __device__ __forceinline__ float get(int) const { return v; }
    __device__ __forceinline__ void set(const float (&f)[1]) { v = f[0]; }
    __device__ __forceinline__ void zero() { v = 0.0f; }
    __device__ __forceinline__ void pin() { pin_vgpr(v); }
};

// V float32 values of a dgamma partial row: 16-byte accesses when V >= 4.
template <int V>
__device__ __forceinline__ void store_f32(float *p, const float (&a)[V])
{
    if constexpr (V % 4 == 0) {
#pragma unroll
        for (int i = 0; i < V; i += 4)
            *reinterpret_cast<float4 *>(p + i) = make_float4(a[i], a[i + 1], a[i + 2], a[i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
            p[i] = a[i];
    }
}

// The same with the nontemporal hint: a partial row written once at the end
// of the backward and read once by the finalizer.
template <int V>
__device__ __forceinline__ void store_f32_nt(float *p, const float (&a)[V])
{
    if constexpr (V % 4 == 0) {
#pragma unroll
        for (int i = 0; i < V; i += 4) {
            const f32x4_t u = {a[i], a[i + 1], a[i + 2], a[i + 3]};
            __builtin_nontemporal_store(u, reinterpret_cast<f32x4_t *>(p + i));
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
            __builtin_nontemporal_store(a[i], p + i);
    }
}

template <int V>
__device__ __forceinline__ void load_f32(const float *p, float (&a)[V])
{
    if constexpr (V % 4 == 0) {
#pragma unroll
        for (int i = 0; i < V; i += 4) {
            const float4 u = *reinterpret_cast<const float4 *>(p + i);
            a[i] = u.x; a[i + 1] = u.y; a[i + 2] = u.z; a[i + 3] = u.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
            a[i] = p[i];
    }
}

// ---- reductions -----------------------------------------------------------

// DPP lane permutations within a 16-lane row (gfx9 encodings).
enum : int {
    kDppQuadXor1 = 0xB1,    // quad_perm [1,0,3,2]
    kDppQuadXor2 = 0x4E,    // quad_perm [2,3,0,1]
    kDppRowHalfMirror = 0x141,
    kDppRowMirror = 0x140,
};
// ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 0x10 (swap 16-lane halves of 32).
constexpr int kSwizzleXor16 = 0x401F;

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of TEAM lanes (8, 16, 32 or 64); every lane of the
// group gets the same total.  The butterfly stays inside the group, so groups
// of a wavefront may be active independently.
template <int TEAM>
__device__ __forceinline__ float team_sum(float v)
{
    static_assert(TEAM == 8 || TEAM == 16 || TEAM == 32 || TEAM == 64, "team size");
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    v += dpp<kDppRowHalfMirror>(v); // lane i <- lane 7-i within each 8: quads combine
    if constexpr (TEAM >= 16)
        v += dpp<kDppRowMirror>(v); // lane i <- lane 15-i: 8-lane halves combine
    if constexpr (TEAM >= 32)
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kSwizzleXor16));
    if constexpr (TEAM == 64) {
        const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
        const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
        v = lo + hi;
    }
    return v;
}

// Maximum that propagates NaN: NaN when either operand is NaN.  fmaxf returns
// the other operand for a NaN, which would hide a NaN output from an amax.
__device__ __forceinline__ float max_nan(float a, float b) { return (a > b || a != a) ? a : b; }

// Maximum over an aligned group of TEAM lanes, by the same exchanges as
// team_sum; NaN in any lane gives NaN.
template <int TEAM>
__device__ __forceinline__ float team_max(float v)
{
    static_assert(TEAM == 8 || TEAM == 16 || TEAM == 32 || TEAM == 64, "team size");
    v = max_nan(v, dpp<kDppQuadXor1>(v));
    v = max_nan(v, dpp<kDppQuadXor2>(v));
    v = max_nan(v, dpp<kDppRowHalfMirror>(v));
    if constexpr (TEAM >= 16)
        v = max_nan(v, dpp<kDppRowMirror>(v));
    if constexpr (TEAM >= 32)
        v = max_nan(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kSwizzleXor16)));
    if constexpr (TEAM == 64) {
        const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
        const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
        v = max_nan(lo, hi);
    }
    return v;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes the compiler wait for every outstanding global load
// (s_waitcnt vmcnt(0)) and so drains the rows a team has in flight; the
// reductions here exchange data through LDS alone.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over the whole workgroup of `threads` lanes (a multiple of 64, at most
// 1024): wavefront sums, then a fixed-order sum of the per-wave totals through
// LDS.  `slot` holds 16 floats; callers alternate between two slots on
// consecutive calls so that one barrier per call suffices.
__device__ __forceinline__ float block_sum(float v, float *slot, int threads)
{
    v = team_sum<64>(v);
    const int nw = threads >> 6;
    if (nw == 1)
        return v;
    if ((threadIdx.x & 63) == 0)
        slot[threadIdx.x >> 6] = v;
    lds_barrier();
    float s = slot[0];
    for (int i = 1; i < nw; ++i)
        s += slot[i];
    return s;
}

// Two sums over the whole workgroup with one barrier (as block_sum; `slot`
// holds 32 floats, callers alternate slots as for block_sum).
__device__ __forceinline__ void block_sum2(float &a, float &b, float *slot, int threads)
{
    a = team_sum<64>(a);
    b = team_sum<64>(b);
    const int nw = threads >> 6;
    if (nw == 1)
        return;
    if ((threadIdx.x & 63) == 0) {
        slot[threadIdx.x >> 6] = a;
        slot[16 + (threadIdx.x >> 6)] = b;
    }
    lds_barrier();
    float sa = slot[0], sb = slot[16];
    for (int i = 1; i < nw; ++i) {
        sa += slot[i];
        sb += slot[16 + i];
    }
    a = sa;
    b = sb;
}

// Four sums over the whole workgroup with one barrier (as block_sum2; `slot`
// holds 64 floats): LayerNorm's two row sums for two rows.
__device__ __forceinline__ void block_sum4(float &a, float &b, float &c, float &d, float *slot, int threads)
{
    a = team_sum<64>(a);
    b = team_sum<64>(b);
    c = team_sum<64>(c);
    d = team_sum<64>(d);
    const int nw = threads >> 6;
    if (nw == 1)
        return;
    if ((threadIdx.x & 63) == 0) {
        const int w = threadIdx.x >> 6;
        slot[w] = a;
        slot[16 + w] = b;
        slot[32 + w] = c;
        slot[48 + w] = d;
    }
    lds_barrier();
    float sa = slot[0], sb = slot[16], sc = slot[32], sd = slot[48];
    for (int i = 1; i < nw; ++i) {
        sa += slot[i];
        sb += slot[16 + i];
        sc += slot[32 + i];
        sd += slot[48 + i];
    }
    a = sa;
    b = sb;
    c = sc;
    d = sd;
}

// Maximum over the whole workgroup, NaN-propagating (as block_sum; `slot`
// holds 16 floats and must not be in use by a concurrent block_sum).
__device__ __forceinline__ float block_max(float v, float *slot, int threads)
{
    v = team_max<64>(v);
    const int nw = threads >> 6;
    if (nw == 1)
        return v;
    if ((threadIdx.x & 63) == 0)
        slot[threadIdx.x >> 6] = v;
    lds_barrier();
    float s = slot[0];
    for (int i = 1; i < nw; ++i)
        s = max_nan(s, slot[i]);
    return s;
}

// ---- fp8 output -----------------------------------------------------------

// OCP E4M3 ("FN") codes of V float32 values times `scale`, nearest even,
// saturating at +-448, written with one store of V bytes (nontemporal like the
// other row outputs).  The gfx950 pack conversion rounds to nearest even but
// turns magnitudes past the format's range into NaN, so finite magnitudes
// beyond 448 (the largest finite code) are clamped first; a NaN passes the
// comparison unchanged and is written as a NaN code.  `am` accumulates max |f|
// (before scaling), NaN-propagating.
template <int V>
__device__ __forceinline__ void store_e4m3(uint8_t *p, const float (&f)[V], float scale, float &am)
{
    float t[V];
    // max |f| over bit patterns: with the sign cleared, unsigned order is
    // numeric order and every NaN lies above +inf, so an integer max
    // propagates NaN in one instruction (am is never negative).  The float
    // form (compare, unordered compare, select) measured 3% slower on the
    // 4096 x 4096 and 16384 x 8192 bf16 fp8 forwards.
    uint32_t m = __builtin_bit_cast(uint32_t, am);
#pragma unroll
    for (int e = 0; e < V; ++e) {
        m = max(m, __builtin_bit_cast(uint32_t, f[e]) & 0x7fffffffu);
        const float s = f[e] * scale;
        t[e] = fabsf(s) > 448.0f ? copysignf(448.0f, s) : s;
    }
    am = __builtin_bit_cast(float, m);
    if constexpr (V == 1) {
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], 0.0f, 0, false);
        __builtin_nontemporal_store((uint8_t)(w & 0xff), p);
    } else if constexpr (V == 4) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false); // bytes 0, 1
        w = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], w, true);       // bytes 2, 3
        __builtin_nontemporal_store((uint32_t)w, reinterpret_cast<uint32_t *>(p));
    } else {
        static_assert(V == 8, "fp8 store of 1, 4 or 8 values");
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(t[4], t[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(t[6], t[7], hi, true);
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t u = {(unsigned)lo, (unsigned)hi};
        __builtin_nontemporal_store(u, reinterpret_cast<u32x2_t *>(p));
    }
}

// ---- row pipeline ---------------------------------------------------------

// A team walks rows row0, row0 + stride, ... < M.  It keeps D rows in flight
// (D = 0: none, for launches where each team owns a single row):
// the loads of row i + D * stride are issued before row i is reduced and
// written, so each row's memory latency overlaps the work on the D rows before
// it.  The D + 1 row buffers form a ring whose indices are compile-time
// constants after unrolling, so the buffers live in VGPRs.
//
// Every load is issued unconditionally: a row index past the team's last row
// is clamped to that last row (a repeat load that hits in cache).  The
// compiler's wait counting does not follow values across branches, so a load
// that may be skipped on some path makes it wait for all outstanding loads
// (s_waitcnt vmcnt(0)), which would drain the rows in flight.  The row test
// is uniform across the team (across the workgroup for workgroup teams), so
// `proc` may contain workgroup barriers.
template <int D, typename Row, typename LoadF, typename ProcF>
__device__ __forceinline__ void row_pipeline(int64_t row0, int64_t stride, int64_t M, LoadF &&load, ProcF &&proc)
{
    if constexpr (D == 0) { // no prefetch: each row is loaded right before it is used
        Row b;
        for (int64_t r = row0; r < M; r += stride) {
            load(b, r);
            proc(b, r);
        }
        return;
    }
    const int64_t last = row0 < M ? row0 + (M - 1 - row0) / stride * stride : M - 1;
    auto clamp = [&](int64_t r) __attribute__((always_inline)) { return r < last ? r : last; };
    Row buf[D + 1];
#pragma unroll
    for (int d = 0; d < D; ++d)
        load(buf[d], clamp(row0 + (int64_t)d * stride));
    for (int64_t base = row0; base < M; base += (int64_t)(D + 1) * stride) {
#pragma unroll
        for (int s = 0; s <= D; ++s) {
            const int64_t r = base + (int64_t)s * stride;
            if (r >= M)
                break;
            load(buf[(s + D) % (D + 1)], clamp(r + (int64_t)D * stride));
            proc(buf[s], r);
        }
    }
}

} // namespace rmsnorm
