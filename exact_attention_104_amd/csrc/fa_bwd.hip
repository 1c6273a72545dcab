// fa_bwd: bf16 attention backward for gfx950 by recomputation.
//
// Method ([HUB] "How it works": store only L_i = m_i + log l_i and recompute
// P_ij = exp(S_ij - L_i) tile by tile; [LIB] "FA1 — changing the order of the
// operations": recomputation in the backward pass). The gradients are those
// of the forward definition: dV = P^T dO, dP = dO V^T, D = rowsum(dO o O),
// dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q.
//
// Two launches on the caller's stream, none with atomics:
//   1. dq_kernel   : (fa_bwd_dq.hip) one workgroup per (batch, head, 256-row Q
//                    block) streaming K / V tiles: S^T, dP^T, dS^T, then
//                    dQ^T += K^T dS^T. Each wave first forms D = rowsum(dO o O)
//                    of its 32 rows in fp32 (it holds their dO already) and
//                    writes it to the workspace for the next launch.
//   2. dkdv_kernel : one workgroup per (batch, head, 128-key block); four waves
//                    own 32 keys each and keep K, V (MFMA operands) and the dK,
//                    dV accumulators in registers for the whole pass. For every
//                    32-row Q block: S = Q K^T and dP = dO V^T (lane = key),
//                    P and dS lane-locally, dV += P^T dO and dK += dS^T Q with
//                    dO / Q read transposed from LDS; software pipelined so
//                    that one block's dV / dK products overlap the next
//                    block's P / dS work. The next blocks' tiles arrive by
//                    direct global->LDS loads meanwhile.
// Splitting dQ from dK/dV recomputes S and dP once more (7 instead of 5
// matrix products) but needs no fp32 atomics: on this chip an fp32 atomic add
// retires about ten times slower than a store, and one dQ partial per
// (key block, query block) pair would cost more than the extra products.
// Every output is written once by one wave, so the results are deterministic.
#include "fa_bwd_impl.h"

namespace fa {

int launch_bwd(const BwdArgs& a) {
  if (a.d == 256) return launch_bwd_d256(a);
  return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

}  // namespace fa
