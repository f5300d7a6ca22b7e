// bf16 dK/dV kernel instances for one head dim and gradient type; compiled
// with -DJ_D=<32|64|128> -DJ_TG=<bf16|f32>.
#include "bwd2_impl.hpp"

#if !defined(J_D) || !defined(J_TG)
#error "J_D and J_TG must be defined"
#endif

namespace jattn {

typedef float f32;

namespace {

template <int D, int WKV, int WKQ, int ACT, bool BIAS, int DBIAS, bool SPLIT, bool WIN = false>
hipError_t dkdv2_one(const BwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((dkdv2_kernel<J_TG, D, WKV, WKQ, ACT, BIAS, DBIAS, SPLIT, WIN>), dim3(grid), dim3(256), 0, st,
                     a);
  return hipGetLastError();
}
// sliding window: 128-key units, 32-query steps, no dBias (softmax without
// split operands at D = 128 runs the wave-pair kernel: not instantiated here)
template <int ACT>
hipError_t dkdv2_window(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.wkv != 4 || k.dbias) return hipErrorInvalidValue;
  if constexpr (J_D == 128 && ACT == kSoftmax) {
    if (!k.split) return hipErrorInvalidValue;
    if (k.bias) return dkdv2_one<J_D, 4, 1, ACT, true, 0, true, true>(a, grid, st);
    return dkdv2_one<J_D, 4, 1, ACT, false, 0, true, true>(a, grid, st);
  } else {
    if (k.bias) return k.split ? dkdv2_one<J_D, 4, 1, ACT, true, 0, true, true>(a, grid, st) : dkdv2_one<J_D, 4, 1, ACT, true, 0, false, true>(a, grid, st);
    return k.split ? dkdv2_one<J_D, 4, 1, ACT, false, 0, true, true>(a, grid, st) : dkdv2_one<J_D, 4, 1, ACT, false, 0, false, true>(a, grid, st);
  }
}

template <int D, int WKV, int WKQ, int ACT, bool SPLIT>
hipError_t dkdv2_bias(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.bias) {
    if (k.dbias && k.dbias_f32) return dkdv2_one<D, WKV, WKQ, ACT, true, 2, SPLIT>(a, grid, st);
    if (k.dbias) return dkdv2_one<D, WKV, WKQ, ACT, true, 1, SPLIT>(a, grid, st);
    return dkdv2_one<D, WKV, WKQ, ACT, true, 0, SPLIT>(a, grid, st);
  }
  return dkdv2_one<D, WKV, WKQ, ACT, false, 0, SPLIT>(a, grid, st);
}

template <int D, int WKV, int WKQ, int ACT>
hipError_t dkdv2_act(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.split) return dkdv2_bias<D, WKV, WKQ, ACT, true>(a, k, grid, st);
  // softmax without split operands on 128-key units at D = 128 runs the
  // wave-pair kernel: not instantiated here
  if constexpr (D == 128 && WKV == 4 && ACT == kSoftmax) return hipErrorInvalidValue;
  else return dkdv2_bias<D, WKV, WKQ, ACT, false>(a, k, grid, st);
}

template <int D, int WKV, int WKQ>
hipError_t dkdv2_shape(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.act == kSoftmax) return dkdv2_act<D, WKV, WKQ, kSoftmax>(a, k, grid, st);
  if (k.act == kGelu) return dkdv2_act<D, WKV, WKQ, kGelu>(a, k, grid, st);
  if (k.act == kGeluPoly) return dkdv2_act<D, WKV, WKQ, kGeluPoly>(a, k, grid, st);
  return dkdv2_act<D, WKV, WKQ, kSilu>(a, k, grid, st);
}

}  // namespace

#define JATTN_DKDV2_NAME_(D, TG) launch_dkdv2_##D##_##TG
#define JATTN_DKDV2_NAME(D, TG) JATTN_DKDV2_NAME_(D, TG)

hipError_t JATTN_DKDV2_NAME(J_D, J_TG)(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.window) {
    if (k.act == kSoftmax) return dkdv2_window<kSoftmax>(a, k, grid, st);
    if (k.act == kGelu) return dkdv2_window<kGelu>(a, k, grid, st);
    if (k.act == kGeluPoly) return dkdv2_window<kGeluPoly>(a, k, grid, st);
    return dkdv2_window<kSilu>(a, k, grid, st);
  }
  if (k.wkv == 4) return dkdv2_shape<J_D, 4, 1>(a, k, grid, st);
  if (k.wkv == 2) return dkdv2_shape<J_D, 2, 2>(a, k, grid, st);
  if constexpr (J_D == 128) {
    // 128-query steps need 73 KB stages at this head dim: fewer than the
    // three the pipeline needs fit in LDS; the planner never selects them
    return hipErrorInvalidValue;
  } else {
    return dkdv2_shape<J_D, 1, 4>(a, k, grid, st);
  }
}

}  // namespace jattn
