// Backward launchers for d = 64 and 128, and the fused variant's dK/dV/dQ
// kernel (the kernels themselves: bwd_kernels.h; d = 256: bwd256.hip, built
// with the compiler's default scheduling strategy, under which its dK/dV
// kernel spills less).
#include "bwd_kernels.h"

namespace attn {

template <bool CAUSAL>
static hipError_t dispatch_bwd(const BwdArgs& a) {
  switch (a.d) {
    case 64: return launch_bwd_t<64, CAUSAL>(a);
    case 128: return launch_bwd_t<128, CAUSAL>(a);
    case 256: return launch_bwd_d256(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a) {
  return a.causal ? dispatch_bwd<true>(a) : dispatch_bwd<false>(a);
}

// The dK/dV kernel with dQ folded in, for the fused backward (bwd_fused.hip
// forms the pairs and clears dqacc before it, and rounds dQ after it); the
// sliding window and the additive bias are template parameters, as in the
// two-kernel backward.
template <int D, bool CAUSAL, bool WIN, bool BIAS>
static hipError_t launch_dkdv_fused_t(const BwdArgs& a, float* dqacc) {
  const int Sqp = (a.Sq + 31) / 32 * 32;
  const int64_t rows_pad = (int64_t)a.B * a.Hq * Sqp;
  const int n_ktiles = (a.Skv + 127) / 128;
  const int BHk = a.B * a.Hkv;
  ATTN_LAUNCH(1, (bwd_dkdv_kernel<D, CAUSAL, WIN, BIAS, true>), dim3(n_ktiles * BHk),
              dim3(256), a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
              (const uint16_t*)a.v, (const uint16_t*)a.d_o, (const float*)a.ws,
              (uint16_t*)a.dk, (uint16_t*)a.dv, BHk, a.Hq, a.Hkv, a.Sq, Sqp, a.Skv, a.window,
              a.bias, a.bias_sb, a.bias_sh, a.scale, a.scale * kLog2e, rows_pad,
              a.Skv - a.Sq, dqacc, 1, nullptr);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv_fused_c(const BwdArgs& a, float* dqacc) {
  if constexpr (CAUSAL) {
    if (a.window > 0)
      return a.bias ? launch_dkdv_fused_t<D, true, true, true>(a, dqacc)
                    : launch_dkdv_fused_t<D, true, true, false>(a, dqacc);
  }
  return a.bias ? launch_dkdv_fused_t<D, CAUSAL, false, true>(a, dqacc)
                : launch_dkdv_fused_t<D, CAUSAL, false, false>(a, dqacc);
}

hipError_t launch_dkdv_fused(const BwdArgs& a, float* dqacc) {
  if (a.d == 64) return a.causal ? launch_dkdv_fused_c<64, true>(a, dqacc)
                                 : launch_dkdv_fused_c<64, false>(a, dqacc);
  if (a.d == 128) return a.causal ? launch_dkdv_fused_c<128, true>(a, dqacc)
                                  : launch_dkdv_fused_c<128, false>(a, dqacc);
  return hipErrorInvalidValue;
}

}  // namespace attn
