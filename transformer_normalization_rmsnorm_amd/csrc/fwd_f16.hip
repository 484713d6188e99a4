// Forward kernel instances for IEEE binary16 storage.
#include "fwd_kernels.h"

namespace rmsnorm {
template hipError_t launch_fwd_typed<f16_t>(bool, FwdKind, const rmsnorm_plan &, const FwdArgs &, hipStream_t);
} // namespace rmsnorm
