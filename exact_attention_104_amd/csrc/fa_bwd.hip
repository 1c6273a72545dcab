// fa_bwd: backward pass (not built yet: every call reports a launch failure).
#include "fa_internal.h"
namespace fa {
int launch_bwd(const BwdArgs&) { return 1; }
}  // namespace fa
