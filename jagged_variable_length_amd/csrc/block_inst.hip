// BlockAttention kernel instances (bf16 inputs; D = 32, 64, 128; with and
// without the fused rotary embedding).
#include "block_impl.hpp"

namespace jattn {

namespace {
template <int D, bool ROPE>
hipError_t fwd_r(const FwdArgs& a, bool out_f32, int grid, hipStream_t st) {
  if (out_f32)
    hipLaunchKernelGGL((block_fwd_kernel<float, D, ROPE>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((block_fwd_kernel<bf16, D, ROPE>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}
template <int D, bool ROPE>
hipError_t bwd_r(const BwdArgs& a, bool grad_f32, int grid, hipStream_t st) {
  if (grad_f32)
    hipLaunchKernelGGL((block_bwd_kernel<float, D, ROPE>), dim3(grid), dim3(kPairThreads), 0, st, a);
  else
    hipLaunchKernelGGL((block_bwd_kernel<bf16, D, ROPE>), dim3(grid), dim3(kPairThreads), 0, st, a);
  return hipGetLastError();
}
template <int D>
hipError_t fwd_d(const FwdArgs& a, bool out_f32, int grid, hipStream_t st) {
  return a.rope_theta ? fwd_r<D, true>(a, out_f32, grid, st) : fwd_r<D, false>(a, out_f32, grid, st);
}
template <int D>
hipError_t bwd_d(const BwdArgs& a, bool grad_f32, int grid, hipStream_t st) {
  return a.rope_theta ? bwd_r<D, true>(a, grad_f32, grid, st) : bwd_r<D, false>(a, grad_f32, grid, st);
}
}  // namespace

hipError_t launch_block_fwd(const FwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.D == 128) return fwd_d<128>(a, k.out_f32, grid, st);
  if (k.D == 64) return fwd_d<64>(a, k.out_f32, grid, st);
  return fwd_d<32>(a, k.out_f32, grid, st);
}

hipError_t launch_block_bwd(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.D == 128) return bwd_d<128>(a, k.out_f32, grid, st);
  if (k.D == 64) return bwd_d<64>(a, k.out_f32, grid, st);
  return bwd_d<32>(a, k.out_f32, grid, st);
}

}  // namespace jattn
