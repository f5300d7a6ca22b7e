// Kernel argument blocks and launchers shared by the host library and the
// device translation units.  Internal to libjattn.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jattn {

// Plan pointers live in the caller's workspace (uploaded by jattn_plan_upload).
struct PlanPtrs {
  const int32_t* units;       // (b, h, tile, cost) per unit, in worker order
  const int32_t* worker_off;  // [W + 1]
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;
  void* o;
  float* lse;
  const int32_t* units;
  const int32_t* worker_off;
  const int32_t* samples;  // 8 int32 per sample
  int H;
  float scale;       // softmax / activation scale
  float scale_log2;  // scale * log2(e)
  int64_t bias_elems;  // elements of the whole bias tensor (bounds its loads)
  int win_l, win_r;    // sliding window: query i sees keys i - win_l .. i + win_r
  const double* rope_theta;  // block mode with RoPE: theta_j, j < D/2 (else null)
};

struct DiArgs {
  const void* o;
  const void* dout;
  float* di;
  int64_t rows;       // Tq * H
  const float* lse;   // [Tq, H] natural log (may be null)
  float* lse2;        // out: lse * log2(e), read by the bf16 backward kernels
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;
  const void* dout;
  const float* lse;  // [Tq, H] natural log
  const float* di;   // [Tq, H]
  const float* lse2; // [Tq, H] lse * log2(e)
  void* dq;
  void* dk;
  void* dv;
  void* dbias;
  const int32_t* units;
  const int32_t* worker_off;
  const int32_t* samples;
  int H;
  float scale;
  float scale_log2;
  int64_t bias_elems;  // elements of the whole bias tensor (bounds its loads)
  int win_l, win_r;    // sliding window: query i sees keys i - win_l .. i + win_r
  const double* rope_theta;  // block mode with RoPE: theta_j, j < D/2 (else null)
  // dQ with the row statistics folded in (bf16 softmax): O (out dtype) and the
  // natural LSE are read, Di and LSE * log2(e) written here for dK/dV
  const void* o;
  float* rs_di;
  float* rs_lse2;
};

// MXFP8 tensor as the kernels see it (see mx_impl.hpp for the layout)
struct MxTensor {
  const uint8_t* codes;    // [T, H, D] E4M3 codes
  const uint8_t* codes_t;  // [RB, H, D, 32] the same, per 32-token block, feature-major
  const uint8_t* scales;   // [RB, H, D/32] E8M0 bytes
};

struct MxQuantArgs {
  const void* x;           // bf16 [T, H, D]
  uint8_t* codes;
  uint8_t* codes_t;        // may be null (not written)
  uint8_t* scales;
  const int32_t* blocks;   // [RB][2]: first row, rows of each 32-row block
  int H;
  int64_t nblocks;
};

struct MxFwdArgs {
  MxTensor q, k, v;
  void* o;
  float* lse;
  const int32_t* units;
  const int32_t* worker_off;
  const int32_t* samples;  // entries 6, 7: first row block of the sample's queries / keys
  int H;
  float scale;
  float scale_log2;
};

struct MxDiArgs {
  MxTensor dout;           // codes, scales of dO
  const void* o;           // out dtype [Tq, H, D]
  const float* lse;        // [Tq, H]
  float* di;               // out [Tq, H]
  float* lse2;             // out [Tq, H]: lse * log2(e)
  const int32_t* blocks;   // [RBq][2] query row blocks
  int H;
  int64_t nblocks;
};

struct MxBwdArgs {
  MxTensor q, k, v, dout;
  const float* di;         // [Tq, H]
  const float* lse2;       // [Tq, H]
  void* dq;
  void* dk;
  void* dv;
  const int32_t* units;
  const int32_t* worker_off;
  const int32_t* samples;
  int H;
  float scale;
  float scale_log2;
};

// Which template instance to run.
struct KernelSel {
  int D;          // 32, 64, 128
  int act;        // 0 softmax, 1 gelu, 2 silu
  bool bias;      // additive bias input
  bool dbias;     // write dBias
  bool dbias_f32; // dBias element type is fp32 (else bf16)
  bool split;     // hi/lo bf16 operands for P / dS products
  bool in_f32;    // inputs are fp32 (else bf16)
  bool out_f32;   // O (fwd) or dQ/dK/dV (bwd) are fp32 (else bf16)
  int wq;         // fwd/dq: waves along queries (4 or 1; 1 => 4-way key split)
  int wkv;        // dkdv: waves along keys (4, 2 or 1; the rest split queries)
  bool window;    // sliding-window mask (bf16 inputs; wq = 4, wkv = 4)
  bool o_f32;     // bwd, softmax: O is fp32 (else bf16)
  bool fold;      // bwd, bf16 softmax: dQ forms Di and LSE*log2e (and runs before dK/dV)
};

#define JATTN_FWD_LAUNCHER_(D, TI, TO) launch_fwd_##D##_##TI##_##TO
#define JATTN_FWD_LAUNCHER(D, TI, TO) JATTN_FWD_LAUNCHER_(D, TI, TO)
#define JATTN_DECLARE_FWD(D, TI, TO) \
  hipError_t JATTN_FWD_LAUNCHER(D, TI, TO)(const FwdArgs&, const KernelSel&, int, hipStream_t);

// fp32 inputs (first-generation kernels); bf16 inputs use launch_fwd2_* below
JATTN_DECLARE_FWD(64, f32, f32)
JATTN_DECLARE_FWD(32, f32, f32)

#define JATTN_BWD_LAUNCHER_(K, D, TI, TG) launch_##K##_##D##_##TI##_##TG
#define JATTN_BWD_LAUNCHER(K, D, TI, TG) JATTN_BWD_LAUNCHER_(K, D, TI, TG)
#define JATTN_DECLARE_BWD(D, TI, TG)                                                                  \
  hipError_t JATTN_BWD_LAUNCHER(dq, D, TI, TG)(const BwdArgs&, const KernelSel&, int, hipStream_t);   \
  hipError_t JATTN_BWD_LAUNCHER(dkdv, D, TI, TG)(const BwdArgs&, const KernelSel&, int, hipStream_t);

// fp32 inputs; bf16 inputs use launch_dkdv2_* / launch_dq2_* below
JATTN_DECLARE_BWD(64, f32, f32)
JATTN_DECLARE_BWD(32, f32, f32)

#define JATTN_DI_LAUNCHER_(D, TI) launch_di_##D##_##TI
#define JATTN_DI_LAUNCHER(D, TI) JATTN_DI_LAUNCHER_(D, TI)
#define JATTN_DECLARE_DI(D, TI) hipError_t JATTN_DI_LAUNCHER(D, TI)(const DiArgs&, bool, hipStream_t);
JATTN_DECLARE_DI(128, bf16)
JATTN_DECLARE_DI(64, bf16)
JATTN_DECLARE_DI(64, f32)
JATTN_DECLARE_DI(32, bf16)
JATTN_DECLARE_DI(32, f32)

// bf16 dK/dV (LDS-DMA pipeline); one translation unit per (head dim, gradient type)
hipError_t launch_dkdv2_128_bf16(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dkdv2_128_f32(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dkdv2_64_bf16(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dkdv2_64_f32(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dkdv2_32_bf16(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dkdv2_32_f32(const BwdArgs&, const KernelSel&, int, hipStream_t);
// wave-pair dK/dV (bf16 inputs, softmax without split operands, dense mask or
// sliding window, 128-key units, D = 128)
hipError_t launch_dkdv_pair_128_bf16(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dkdv_pair_128_f32(const BwdArgs&, const KernelSel&, int, hipStream_t);

// bf16 dQ (LDS-DMA pipeline); one translation unit per (head dim, gradient type)
hipError_t launch_dq2_128_bf16(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dq2_128_f32(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dq2_64_bf16(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dq2_64_f32(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dq2_32_bf16(const BwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_dq2_32_f32(const BwdArgs&, const KernelSel&, int, hipStream_t);

// bf16 forward (LDS-DMA pipeline); one translation unit per head dim
hipError_t launch_fwd2_128(const FwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_fwd2_64(const FwdArgs&, const KernelSel&, int, hipStream_t);
hipError_t launch_fwd2_32(const FwdArgs&, const KernelSel&, int, hipStream_t);

hipError_t launch_fwd(const FwdArgs& a, const KernelSel& k, int grid, hipStream_t st);
hipError_t launch_dq(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st);
hipError_t launch_dkdv(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st);
hipError_t launch_di(const DiArgs& a, const KernelSel& k, bool o_f32, hipStream_t st);
// BlockAttention: grid = number of workgroups; each workgroup runs two
// workers (wave pairs) of the block plan.
hipError_t launch_block_fwd(const FwdArgs& a, const KernelSel& k, int grid, hipStream_t st);
hipError_t launch_block_bwd(const BwdArgs& a, const KernelSel& k, int grid, hipStream_t st);

// MXFP8 (mx_inst.hip, one translation unit per head dim)
hipError_t launch_mx_quant_128(const MxQuantArgs&, hipStream_t);
hipError_t launch_mx_quant_64(const MxQuantArgs&, hipStream_t);
hipError_t launch_mx_fwd_128(const MxFwdArgs&, int act, bool out_f32, int grid, hipStream_t);
hipError_t launch_mx_fwd_64(const MxFwdArgs&, int act, bool out_f32, int grid, hipStream_t);
hipError_t launch_mx_di_128(const MxDiArgs&, bool o_f32, hipStream_t);
hipError_t launch_mx_di_64(const MxDiArgs&, bool o_f32, hipStream_t);
hipError_t launch_mx_dkdv_128(const MxBwdArgs&, int act, bool grad_f32, int grid, hipStream_t);
hipError_t launch_mx_dkdv_64(const MxBwdArgs&, int act, bool grad_f32, int grid, hipStream_t);
hipError_t launch_mx_dq_128(const MxBwdArgs&, int act, bool grad_f32, int grid, hipStream_t);
hipError_t launch_mx_dq_64(const MxBwdArgs&, int act, bool grad_f32, int grid, hipStream_t);

// Fixed device scratch (fixed_scratch.hip): its size, and its address on the
// current device (looked up on the first call per device, then kept).
size_t fixed_scratch_bytes();
hipError_t fixed_scratch_address(void** out);

// QK-norm (row-wise L2 normalisation) of `rows` rows of D elements
hipError_t launch_l2norm_fwd(const void* x, void* y, float* rnorm, int64_t rows, int D, bool x_f32, bool y_f32,
                             hipStream_t st);
hipError_t launch_l2norm_bwd(const void* x, const void* dy, void* dx, int64_t rows, int D, bool x_f32, bool dy_f32,
                             bool dx_f32, hipStream_t st);

}  // namespace jattn
