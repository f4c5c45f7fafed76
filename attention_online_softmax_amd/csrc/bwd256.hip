// Backward launchers for d = 256: the kernels of bwd_kernels.h at one wave
// per SIMD (their dK and dV accumulators alone take 256 registers per lane),
// in a translation unit of their own so that they are compiled with the
// default scheduling strategy (the d = 64 and 128 kernels in bwd.hip use the
// iterative ILP strategy, under which the d = 256 dK/dV kernel spills more).
#include "bwd_kernels.h"

namespace attn {

hipError_t launch_bwd_d256(const BwdArgs& a) {
  return a.causal ? launch_bwd_t<256, true>(a) : launch_bwd_t<256, false>(a);
}

}  // namespace attn
