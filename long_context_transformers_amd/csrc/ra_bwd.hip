// ra_bwd.hip -- block backward of Ring Attention on gfx950.
#include "ra_internal.h"

namespace ra {

hipError_t launch_bwd(const BwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ra
