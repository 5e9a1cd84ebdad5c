// Dispatch of the bf16 forward to the tile width that holds a row: the
// smallest of 64, 96, 128, 192 and 256 at least the head size (shorter rows are
// padded in the tiles).  Each width is compiled in its own translation unit.
#include "fa_kernels.h"

namespace fa {

hipError_t launch_fwd_w64(const FwdArgs& a);
hipError_t launch_fwd_w96(const FwdArgs& a);
hipError_t launch_fwd_w128(const FwdArgs& a);
hipError_t launch_fwd_w192(const FwdArgs& a);
hipError_t launch_fwd_w256(const FwdArgs& a);

hipError_t launch_fwd_bf16(const FwdArgs& a) {
    if (a.d <= 64) return launch_fwd_w64(a);
    if (a.d <= 96) return launch_fwd_w96(a);
    if (a.d <= 128) return launch_fwd_w128(a);
    if (a.d <= 192) return launch_fwd_w192(a);
    return launch_fwd_w256(a);
}

}  // namespace fa
