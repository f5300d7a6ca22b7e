// One translation unit per (head dim, input type, gradient type) of the
// fp32-input backward kernels, compiled with -DJ_D=<32|64> -DJ_TI=f32
// -DJ_TG=f32, plus the Di pass (-DJ_DI).  For bf16 inputs only the Di pass is
// built from here (-DJ_DI -DJ_DI_ONLY): their dK/dV and dQ kernels are the
// LDS-DMA ones of bwd2_inst.hip and dq2_inst.hip.
#include "bwd_impl.hpp"

#ifndef J_D
#error "J_D must be defined"
#endif

namespace jattn {

typedef float f32;

#ifndef J_DI_ONLY
namespace {

template <typename TI, typename TG, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT>
hipError_t dq_one(const BwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((dq_kernel<TI, TG, D, WQ, WK, ACT, BIAS, SPLIT>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename TI, typename TG, int D, int WQ, int WK, int ACT>
hipError_t dq_act(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  constexpr bool kCanSplit = sizeof(TI) == 2;
  const bool split = kCanSplit && k.split;
  if (k.bias) {
    if (split) return dq_one<TI, TG, D, WQ, WK, ACT, true, kCanSplit>(a, grid, st);
    return dq_one<TI, TG, D, WQ, WK, ACT, true, false>(a, grid, st);
  }
  if (split) return dq_one<TI, TG, D, WQ, WK, ACT, false, kCanSplit>(a, grid, st);
  return dq_one<TI, TG, D, WQ, WK, ACT, false, false>(a, grid, st);
}

template <typename TI, typename TG, int D, int WQ, int WK>
hipError_t dq_shape(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.act == kSoftmax) return dq_act<TI, TG, D, WQ, WK, kSoftmax>(a, k, grid, st);
  if (k.act == kGelu) return dq_act<TI, TG, D, WQ, WK, kGelu>(a, k, grid, st);
  return dq_act<TI, TG, D, WQ, WK, kSilu>(a, k, grid, st);
}

template <typename TI, typename TG, int D, int WKV, int ACT, bool BIAS, int DBIAS, bool SPLIT>
hipError_t dkdv_one(const BwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((dkdv_kernel<TI, TG, D, WKV, ACT, BIAS, DBIAS, SPLIT>), dim3(grid), dim3(kThreads), 0,
                     st, a);
  return hipGetLastError();
}

template <typename TI, typename TG, int D, int WKV, int ACT, bool SPLIT>
hipError_t dkdv_bias(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.bias) {
    if (k.dbias && k.dbias_f32) return dkdv_one<TI, TG, D, WKV, ACT, true, 2, SPLIT>(a, grid, st);
    if (k.dbias) return dkdv_one<TI, TG, D, WKV, ACT, true, 1, SPLIT>(a, grid, st);
    return dkdv_one<TI, TG, D, WKV, ACT, true, 0, SPLIT>(a, grid, st);
  }
  return dkdv_one<TI, TG, D, WKV, ACT, false, 0, SPLIT>(a, grid, st);
}

template <typename TI, typename TG, int D, int WKV, int ACT>
hipError_t dkdv_act(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  constexpr bool kCanSplit = sizeof(TI) == 2;
  if (kCanSplit && k.split) return dkdv_bias<TI, TG, D, WKV, ACT, kCanSplit>(a, k, grid, st);
  return dkdv_bias<TI, TG, D, WKV, ACT, false>(a, k, grid, st);
}

template <typename TI, typename TG, int D, int WKV>
hipError_t dkdv_shape(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.act == kSoftmax) return dkdv_act<TI, TG, D, WKV, kSoftmax>(a, k, grid, st);
  if (k.act == kGelu) return dkdv_act<TI, TG, D, WKV, kGelu>(a, k, grid, st);
  return dkdv_act<TI, TG, D, WKV, kSilu>(a, k, grid, st);
}

}  // namespace

hipError_t JATTN_BWD_LAUNCHER(dq, J_D, J_TI, J_TG)(const BwdArgs& a, const KernelSel& k, int grid,
                                                    hipStream_t st) {
  if (k.wq == 4) return dq_shape<J_TI, J_TG, J_D, 4, 1>(a, k, grid, st);
  return dq_shape<J_TI, J_TG, J_D, 1, 4>(a, k, grid, st);
}

hipError_t JATTN_BWD_LAUNCHER(dkdv, J_D, J_TI, J_TG)(const BwdArgs& a, const KernelSel& k, int grid,
                                                      hipStream_t st) {
  if (k.wkv == 4) return dkdv_shape<J_TI, J_TG, J_D, 4>(a, k, grid, st);
  if (k.wkv == 2) return dkdv_shape<J_TI, J_TG, J_D, 2>(a, k, grid, st);
  return dkdv_shape<J_TI, J_TG, J_D, 1>(a, k, grid, st);
}
#endif  // J_DI_ONLY

#ifdef J_DI
// Di for this (D, dO type), both O types.
hipError_t JATTN_DI_LAUNCHER(J_D, J_TI)(const DiArgs& a, bool o_f32, hipStream_t st) {
  constexpr int CE = 16 / (int)sizeof(J_TI);
  constexpr int RPB = kThreads / (J_D / CE);
  const int grid = (int)((a.rows + RPB - 1) / RPB);
  if (grid == 0) return hipSuccess;
  if (o_f32)
    hipLaunchKernelGGL((di_kernel<float, J_TI, J_D>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((di_kernel<bf16, J_TI, J_D>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}
#endif

}  // namespace jattn
