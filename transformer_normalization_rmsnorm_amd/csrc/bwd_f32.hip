// Backward and finalizer kernel instances for float32 storage.
#include "bwd_kernels.h"

namespace rmsnorm {
template hipError_t launch_bwd_typed<float>(bool, bool, const rmsnorm_plan &, const BwdArgs &, hipStream_t);
template hipError_t launch_finalize_typed<float>(const float *, int64_t, int64_t, int64_t, void *, void *, hipStream_t);
} // namespace rmsnorm
