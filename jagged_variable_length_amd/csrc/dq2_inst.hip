// bf16 dQ kernel instances for one head dim and gradient type; compiled with
// -DJ_D=<32|64|128> -DJ_TG=<bf16|f32>.
#include "dq2_impl.hpp"

#if !defined(J_D) || !defined(J_TG)
#error "J_D and J_TG must be defined"
#endif

namespace jattn {

typedef float f32;

namespace {

template <int WQ, int WK, int ACT, bool BIAS, bool SPLIT, bool WIN = false, int OF = 0>
hipError_t dq2_launch(const BwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((dq2_kernel<J_TG, J_D, WQ, WK, ACT, BIAS, SPLIT, WIN, OF>), dim3(grid), dim3(64 * WQ * WK), 0,
                     st, a);
  return hipGetLastError();
}
// softmax: dQ forms Di and LSE * log2(e) itself (k.fold) from bf16 O, or from
// fp32 O below D = 128; at D = 128 fp32 O does not fit the registers beside
// the unit's other operands, and those plans keep the separate Di pass
template <int WQ, int WK, int ACT, bool BIAS, bool SPLIT, bool WIN = false>
hipError_t dq2_one(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if constexpr (ACT == kSoftmax) {
    if (!k.fold) {
      if constexpr (J_D == 128) return dq2_launch<WQ, WK, ACT, BIAS, SPLIT, WIN, 0>(a, grid, st);
      return hipErrorInvalidValue;
    }
    if (k.o_f32) {
      if constexpr (J_D < 128) return dq2_launch<WQ, WK, ACT, BIAS, SPLIT, WIN, 2>(a, grid, st);
      return hipErrorInvalidValue;
    }
    return dq2_launch<WQ, WK, ACT, BIAS, SPLIT, WIN, 1>(a, grid, st);
  } else {
    return dq2_launch<WQ, WK, ACT, BIAS, SPLIT, WIN>(a, grid, st);
  }
}
// sliding window: 128-row query tiles, 64-key steps only
template <int ACT>
hipError_t dq2_window(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.wq != 4) return hipErrorInvalidValue;
  if (k.bias) return k.split ? dq2_one<4, 2, ACT, true, true, true>(a, k, grid, st) : dq2_one<4, 2, ACT, true, false, true>(a, k, grid, st);
  return k.split ? dq2_one<4, 2, ACT, false, true, true>(a, k, grid, st) : dq2_one<4, 2, ACT, false, false, true>(a, k, grid, st);
}

template <int WQ, int WK, int ACT>
hipError_t dq2_act(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if constexpr (J_D == 128 && WQ == 1) {
    // a 128-key step leaves no room for a bias tile at this head dim
    if (k.bias) return hipErrorInvalidValue;
  } else if (k.bias) {
    if (k.split) return dq2_one<WQ, WK, ACT, true, true>(a, k, grid, st);
    return dq2_one<WQ, WK, ACT, true, false>(a, k, grid, st);
  }
  if (k.split) return dq2_one<WQ, WK, ACT, false, true>(a, k, grid, st);
  return dq2_one<WQ, WK, ACT, false, false>(a, k, grid, st);
}

template <int WQ, int WK>
hipError_t dq2_shape(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.act == kSoftmax) return dq2_act<WQ, WK, kSoftmax>(a, k, grid, st);
  if (k.act == kGelu) return dq2_act<WQ, WK, kGelu>(a, k, grid, st);
  if (k.act == kGeluPoly) return dq2_act<WQ, WK, kGeluPoly>(a, k, grid, st);
  return dq2_act<WQ, WK, kSilu>(a, k, grid, st);
}

}  // namespace

#define JATTN_DQ2_NAME_(D, TG) launch_dq2_##D##_##TG
#define JATTN_DQ2_NAME(D, TG) JATTN_DQ2_NAME_(D, TG)

hipError_t JATTN_DQ2_NAME(J_D, J_TG)(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st) {
  if (k.window) {
    if (k.act == kSoftmax) return dq2_window<kSoftmax>(a, k, grid, st);
    if (k.act == kGelu) return dq2_window<kGelu>(a, k, grid, st);
    if (k.act == kGeluPoly) return dq2_window<kGeluPoly>(a, k, grid, st);
    return dq2_window<kSilu>(a, k, grid, st);
  }
  if (k.wq == 8) return dq2_shape<8, 1>(a, k, grid, st);
  if constexpr (J_D == 128) {
    // 4 query groups over one 32-key block per step, two workgroups per CU
    // (softmax without a bias or split operands)
    if (k.wq == 4) {
      if (k.bias || k.split || k.act != kSoftmax) return hipErrorInvalidValue;
      return dq2_one<4, 1, kSoftmax, false, false>(a, k, grid, st);
    }
  } else {
    // the same shape, two workgroups per CU (softmax without a bias)
    if (k.wq == 4) {
      if (k.bias || k.act != kSoftmax) return hipErrorInvalidValue;
      if (k.split) return dq2_one<4, 1, kSoftmax, false, true>(a, k, grid, st);
      return dq2_one<4, 1, kSoftmax, false, false>(a, k, grid, st);
    }
  }
  if (k.wq != 1) return hipErrorInvalidValue;  // 4 x 2 serves the windowed instances only
  return dq2_shape<1, 4>(a, k, grid, st);
}

}  // namespace jattn
