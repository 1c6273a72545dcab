// fa_bwd at d = 256: the kernels of fa_bwd_impl.h instantiated for d = 256 in
// a translation unit of their own, built with every MFMA in its VGPR form
// (-mllvm -amdgpu-mfma-vgpr-form, set for this file in build.py). The dK/dV
// kernel then keeps its accumulators, S and dP in VGPRs and its K / V
// operands in AGPRs, which measured faster than the AGPR form at d = 256 and
// slower at d = 128.
#include "fa_bwd_impl.h"

namespace fa {

int launch_bwd_d256(const BwdArgs& a) { return launch_d<256>(a); }

}  // namespace fa
