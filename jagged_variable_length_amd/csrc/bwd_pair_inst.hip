// Wave-pair dK/dV kernel instances (bf16 inputs, softmax, dense mask or
// sliding window, 128-key units) for one head dim and gradient type; compiled with -DJ_D=<64|128>
// -DJ_TG=<bf16|f32>.
#include "bwd_pair_impl.hpp"

#if !defined(J_D) || !defined(J_TG)
#error "J_D and J_TG must be defined"
#endif

namespace jattn {

typedef float f32;

namespace {

template <bool BIAS, int DBIAS, bool WIN = false>
hipError_t pair_one(const BwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((dkdv_pair_kernel<J_TG, J_D, BIAS, DBIAS, WIN>), dim3(grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace

#define JATTN_PAIR_NAME_(D, TG) launch_dkdv_pair_##D##_##TG
#define JATTN_PAIR_NAME(D, TG) JATTN_PAIR_NAME_(D, TG)

hipError_t JATTN_PAIR_NAME(J_D, J_TG)(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.act != kSoftmax || k.split || k.wkv != 4) return hipErrorInvalidValue;
  if (k.window) {
    if (k.dbias) return hipErrorInvalidValue;
    return k.bias ? pair_one<true, 0, true>(a, grid, st) : pair_one<false, 0, true>(a, grid, st);
  }
  if (!k.bias) return pair_one<false, 0>(a, grid, st);
  if (!k.dbias) return pair_one<true, 0>(a, grid, st);
  return k.dbias_f32 ? pair_one<true, 2>(a, grid, st) : pair_one<true, 1>(a, grid, st);
}

}  // namespace jattn
