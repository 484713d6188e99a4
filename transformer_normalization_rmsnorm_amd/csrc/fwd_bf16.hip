// Forward kernel instances for bfloat16 storage.
#include "fwd_kernels.h"

namespace rmsnorm {
template hipError_t launch_fwd_typed<bf16_t>(bool, FwdKind, const rmsnorm_plan &, const FwdArgs &, hipStream_t);
} // namespace rmsnorm
