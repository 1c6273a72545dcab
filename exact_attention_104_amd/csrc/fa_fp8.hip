// fp8 path (not built yet: every call reports a launch failure).
#include "fa_internal.h"
namespace fa {
int launch_quant_fp8(const QuantArgs&) { return 1; }
int launch_fwd_fp8(const Fp8FwdArgs&) { return 1; }
}  // namespace fa
