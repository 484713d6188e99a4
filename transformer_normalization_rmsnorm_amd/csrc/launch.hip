// Storage-type dispatch of the kernel launches, and the fp8 amax finalizer.
//
// The forward and backward kernels are templates over the storage type
// (fwd_kernels.h, bwd_kernels.h); each type's instances live in a unit of its
// own (fwd_bf16.hip, fwd_f16.hip, fwd_f32.hip and the bwd_ units), and the
// functions here pick the unit from the dtype code of the call.
#include "device_common.h"
#include "rmsnorm_internal.h"

namespace rmsnorm {

hipError_t launch_fwd(int dtype, bool fused, FwdKind kind, const rmsnorm_plan &p, const FwdArgs &a, hipStream_t s)
{
    switch (dtype) {
    case RMSNORM_BF16: return launch_fwd_typed<bf16_t>(fused, kind, p, a, s);
    case RMSNORM_F16: return launch_fwd_typed<f16_t>(fused, kind, p, a, s);
    case RMSNORM_F32: return launch_fwd_typed<float>(fused, kind, p, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd(int dtype, bool fused, bool ln, const rmsnorm_plan &p, const BwdArgs &a, hipStream_t s)
{
    switch (dtype) {
    case RMSNORM_BF16: return launch_bwd_typed<bf16_t>(fused, ln, p, a, s);
    case RMSNORM_F16: return launch_bwd_typed<f16_t>(fused, ln, p, a, s);
    case RMSNORM_F32: return launch_bwd_typed<float>(fused, ln, p, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_finalize(int dtype, const float *partials, int64_t programs, int64_t ld, int64_t N,
                           void *dgamma, void *dbeta, hipStream_t s)
{
    switch (dtype) {
    case RMSNORM_BF16: return launch_finalize_typed<bf16_t>(partials, programs, ld, N, dgamma, dbeta, s);
    case RMSNORM_F16: return launch_finalize_typed<f16_t>(partials, programs, ld, N, dgamma, dbeta, s);
    case RMSNORM_F32: return launch_finalize_typed<float>(partials, programs, ld, N, dgamma, dbeta, s);
    default: return hipErrorInvalidValue;
    }
}

// *amax = max(*amax, max_p part[p]), one workgroup; a NaN in any partial (or
// in *amax) gives NaN.  The partials are read as
// float4 with kAmaxLoads independent loads per lane in flight, so a round
// covers kAmaxThreads * kAmaxLoads * 4 partials for one memory latency (a
// dependent loop of scalar loads cost one latency per 256 partials: about 20
// us at 16384 workgroups).  Lanes past the end load nothing: re-reading the
// last group there kept this one compute unit's load path busy for loads
// whose values were ignored (4096 x 4096 fp8 forward 14.46 -> 14.30 us).
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
            v[u] = i < P4 ? p4[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < kAmaxLoads; ++u) {
            const int64_t i = b + (int64_t)u * kAmaxThreads + threadIdx.x;
            if (i < P4)
                m = max_nan(m, max_nan(max_nan(v[u].x, v[u].y), max_nan(v[u].z, v[u].w)));
        }
    }
    for (int64_t i = P4 * 4 + threadIdx.x; i < P; i += kAmaxThreads)
        m = max_nan(m, part[i]);
    m = block_max(m, slot, kAmaxThreads);
    if (threadIdx.x == 0)
        *amax = max_nan(*amax, m);
}

hipError_t launch_amax_finalize(const float *part, int64_t programs, float *amax, hipStream_t s)
{
    hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kAmaxThreads), 0, s, part, programs, amax);
    return hipGetLastError();
}

} // namespace rmsnorm
