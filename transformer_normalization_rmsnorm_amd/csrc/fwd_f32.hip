// Forward kernel instances for float32 storage.
#include "fwd_kernels.h"

namespace rmsnorm {
template hipError_t launch_fwd_typed<float>(bool, FwdKind, const rmsnorm_plan &, const FwdArgs &, hipStream_t);
} // namespace rmsnorm
