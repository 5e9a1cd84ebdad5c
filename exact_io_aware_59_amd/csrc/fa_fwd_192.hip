// Instantiation of the bf16 forward for 192-wide tiles (rows of 144 to 192
// elements); the kernel and its launch logic are in fa_fwd.h.
#include "fa_fwd.h"

namespace fa {

hipError_t launch_fwd_w192(const FwdArgs& a) { return launch_fwd_width<192>(a); }
unsigned debug_flags_fwd_w192(bool clear) { return read_debug_flags(clear); }

}  // namespace fa
