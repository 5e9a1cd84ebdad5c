// Instantiation of the bf16 forward for 96-wide tiles (rows of 80 or 96
// elements); the kernel and its launch logic are in fa_fwd.h.
#include "fa_fwd.h"

namespace fa {

hipError_t launch_fwd_w96(const FwdArgs& a) { return launch_fwd_width<96>(a); }
unsigned debug_flags_fwd_w96(bool clear) { return read_debug_flags(clear); }

}  // namespace fa
