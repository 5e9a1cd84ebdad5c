// Instantiation of the bf16 forward for 256-wide tiles (rows of up to 256
// elements); the kernel and its launch logic are in fa_fwd.h.
#include "fa_fwd.h"

namespace fa {

hipError_t launch_fwd_w256(const FwdArgs& a) { return launch_fwd_width<256>(a); }
unsigned debug_flags_fwd_w256(bool clear) { return read_debug_flags(clear); }

}  // namespace fa
