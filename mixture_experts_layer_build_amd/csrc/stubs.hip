// Entry points whose kernels are not built yet report "unsupported".
#include "mok_internal.h"

namespace mok {
hipError_t launch_backward(mok_workspace*, const void*, const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mok
