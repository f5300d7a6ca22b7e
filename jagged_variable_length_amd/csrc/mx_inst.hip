// MXFP8 kernels for one head dim, compiled with -DJ_D=<64|128>: the
// quantiser, the forward and the backward (softmax, erf-GELU, SiLU; bf16 or
// fp32 outputs and gradients).
#include "mx_bwd_impl.hpp"

#ifndef J_D
#error "J_D must be defined"
#endif

#define MX_CAT_(a, b) a##b
#define MX_CAT(a, b) MX_CAT_(a, b)

namespace jattn {

hipError_t MX_CAT(launch_mx_quant_, J_D)(const MxQuantArgs& a, hipStream_t st) {
  const int64_t grid = a.nblocks * a.H;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((mx_quant_kernel<J_D>), dim3((unsigned)grid), dim3(2 * J_D), 0, st, a);
  return hipGetLastError();
}

namespace {
template <typename TO, int ACT>
hipError_t mx_fwd_one(const MxFwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((mx_fwd_kernel<TO, J_D, ACT>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <typename TO>
hipError_t mx_fwd_act(const MxFwdArgs& a, int act, int grid, hipStream_t st) {
  if (act == kSoftmax) return mx_fwd_one<TO, kSoftmax>(a, grid, st);
  if (act == kGelu) return mx_fwd_one<TO, kGelu>(a, grid, st);
  return mx_fwd_one<TO, kSilu>(a, grid, st);
}
}  // namespace

hipError_t MX_CAT(launch_mx_fwd_, J_D)(const MxFwdArgs& a, int act, bool out_f32, int grid, hipStream_t st) {
  if (out_f32) return mx_fwd_act<float>(a, act, grid, st);
  return mx_fwd_act<bf16>(a, act, grid, st);
}

hipError_t MX_CAT(launch_mx_di_, J_D)(const MxDiArgs& a, bool o_f32, hipStream_t st) {
  const int64_t grid = a.nblocks * a.H;
  if (grid == 0) return hipSuccess;
  if (o_f32)
    hipLaunchKernelGGL((mx_di_kernel<float, J_D>), dim3((unsigned)grid), dim3(2 * J_D), 0, st, a);
  else
    hipLaunchKernelGGL((mx_di_kernel<bf16, J_D>), dim3((unsigned)grid), dim3(2 * J_D), 0, st, a);
  return hipGetLastError();
}

namespace {
template <typename TG, int ACT>
hipError_t mx_bwd_one(const MxBwdArgs& a, bool dq, int grid, hipStream_t st) {
  if (dq)
    hipLaunchKernelGGL((mx_dq_kernel<TG, J_D, ACT>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((mx_dkdv_kernel<TG, J_D, ACT>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <typename TG>
hipError_t mx_bwd_act(const MxBwdArgs& a, int act, bool dq, int grid, hipStream_t st) {
  if (act == kSoftmax) return mx_bwd_one<TG, kSoftmax>(a, dq, grid, st);
  if (act == kGelu) return mx_bwd_one<TG, kGelu>(a, dq, grid, st);
  return mx_bwd_one<TG, kSilu>(a, dq, grid, st);
}
}  // namespace

hipError_t MX_CAT(launch_mx_dkdv_, J_D)(const MxBwdArgs& a, int act, bool grad_f32, int grid, hipStream_t st) {
  return grad_f32 ? mx_bwd_act<float>(a, act, false, grid, st) : mx_bwd_act<bf16>(a, act, false, grid, st);
}

hipError_t MX_CAT(launch_mx_dq_, J_D)(const MxBwdArgs& a, int act, bool grad_f32, int grid, hipStream_t st) {
  return grad_f32 ? mx_bwd_act<float>(a, act, true, grid, st) : mx_bwd_act<bf16>(a, act, true, grid, st);
}

}  // namespace jattn
