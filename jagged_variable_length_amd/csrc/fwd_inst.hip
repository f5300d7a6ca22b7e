// One translation unit per (head dim, input type, output type) of the
// forward kernel; the build compiles this file once per combination with
// -DJ_D=<32|64|128> -DJ_TI=<bf16|f32> -DJ_TO=<bf16|f32>.
#include "fwd_impl.hpp"

#ifndef J_D
#error "J_D must be defined"
#endif

namespace jattn {

typedef float f32;

template <typename TI, typename TO, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT>
static hipError_t launch_one(const FwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<TI, TO, D, WQ, WK, ACT, BIAS, SPLIT>), dim3(grid), dim3(kThreads), 0,
                     st, a);
  return hipGetLastError();
}

template <typename TI, typename TO, int D, int WQ, int WK>
static hipError_t launch_shape(const FwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  constexpr bool kCanSplit = sizeof(TI) == 2;  // hi/lo split only for bf16 operands
  if (k.act == kSoftmax) {
    if (k.bias) return launch_one<TI, TO, D, WQ, WK, kSoftmax, true, false>(a, grid, st);
    return launch_one<TI, TO, D, WQ, WK, kSoftmax, false, false>(a, grid, st);
  }
  const bool split = kCanSplit && k.split;
  if (k.act == kGelu) {
    if (k.bias) {
      if (split) return launch_one<TI, TO, D, WQ, WK, kGelu, true, kCanSplit>(a, grid, st);
      return launch_one<TI, TO, D, WQ, WK, kGelu, true, false>(a, grid, st);
    }
    if (split) return launch_one<TI, TO, D, WQ, WK, kGelu, false, kCanSplit>(a, grid, st);
    return launch_one<TI, TO, D, WQ, WK, kGelu, false, false>(a, grid, st);
  }
  if (k.bias) {
    if (split) return launch_one<TI, TO, D, WQ, WK, kSilu, true, kCanSplit>(a, grid, st);
    return launch_one<TI, TO, D, WQ, WK, kSilu, true, false>(a, grid, st);
  }
  if (split) return launch_one<TI, TO, D, WQ, WK, kSilu, false, kCanSplit>(a, grid, st);
  return launch_one<TI, TO, D, WQ, WK, kSilu, false, false>(a, grid, st);
}

hipError_t JATTN_FWD_LAUNCHER(J_D, J_TI, J_TO)(const FwdArgs& a, const KernelSel& k, int grid,
                                                hipStream_t st) {
  if (k.wq == 4) return launch_shape<J_TI, J_TO, J_D, 4, 1>(a, k, grid, st);
  return launch_shape<J_TI, J_TO, J_D, 1, 4>(a, k, grid, st);
}

}  // namespace jattn
