// Backward and finalizer kernel instances for bfloat16 storage.
#include "bwd_kernels.h"

namespace rmsnorm {
template hipError_t launch_bwd_typed<bf16_t>(bool, bool, const rmsnorm_plan &, const BwdArgs &, hipStream_t);
template hipError_t launch_finalize_typed<bf16_t>(const float *, int64_t, int64_t, int64_t, void *, void *, hipStream_t);
} // namespace rmsnorm
