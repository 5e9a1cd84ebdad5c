// Instantiation of the bf16 forward for 64-wide tiles (rows of up to 64
// elements); the kernel and its launch logic are in fa_fwd.h.
#include "fa_fwd.h"

namespace fa {

hipError_t launch_fwd_w64(const FwdArgs& a) { return launch_fwd_width<64>(a); }

}  // namespace fa
