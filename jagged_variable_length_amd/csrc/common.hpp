// Device-side building blocks shared by the jagged attention kernels.
// gfx950 (CDNA4) only: wave64, MFMA 32x32 tiles, raw buffer loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jattn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // four waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// activation codes (match the public header)
constexpr int kSoftmax = 0;
constexpr int kGelu = 1;
constexpr int kSilu = 2;
constexpr int kGeluPoly = 3;

// ---------------------------------------------------------------------------
// Sample table entry as uploaded by the host: {q0, lq, k0, lk, bias_lo,
// bias_hi, 0, 0} (int32).  q0/k0 are the first rows of the sample.
// ---------------------------------------------------------------------------
struct Sample {
  int q0, lq, k0, lk;
  int64_t bias0;
};

__device__ __forceinline__ Sample load_sample(const int32_t* table, int b) {
  const i32x4* p = reinterpret_cast<const i32x4*>(table + 8 * b);
  i32x4 a = p[0];
  i32x4 c = p[1];
  Sample s;
  s.q0 = __builtin_amdgcn_readfirstlane(a[0]);
  s.lq = __builtin_amdgcn_readfirstlane(a[1]);
  s.k0 = __builtin_amdgcn_readfirstlane(a[2]);
  s.lk = __builtin_amdgcn_readfirstlane(a[3]);
  s.bias0 = (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane(c[0]) |
            ((int64_t)__builtin_amdgcn_readfirstlane(c[1]) << 32);
  return s;
}

// Worker index for workgroup blockIdx.x.  Hardware dispatches consecutive
// workgroups round-robin over the 8 XCDs; this maps consecutive workers to
// one XCD so that neighbouring units (same sample/head after the cost sort)
// share that XCD's L2.
__device__ __forceinline__ int xcd_worker(int block, int nblocks) {
  if ((nblocks & 7) != 0) return block;
  return (block & 7) * (nblocks >> 3) + (block >> 3);
}

// ---------------------------------------------------------------------------
// Raw buffer resources: loads at or past num_records bytes return zero.  This
// is how tail rows of a sample read as zero without any per-element test.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Every call site passes a per-unit (wave-uniform) base and size; reading
// them through readfirstlane lets the descriptor live in SGPRs, as buffer
// instructions require, instead of a per-lane loop over descriptors.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* q = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  // word 3 = 0x00020000: 32-bit data format for raw (untyped) access on gfx9
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Unit record (b, h, tile, cost), read once per wave and kept in SGPRs.
__device__ __forceinline__ i32x4 load_unit(const int32_t* units, int u) {
  const i32x4 x = reinterpret_cast<const i32x4*>(units)[u];
  return i32x4{uniform(x[0]), uniform(x[1]), uniform(x[2]), uniform(x[3])};
}

__device__ __forceinline__ i32x4 buf_load16(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}
__device__ __forceinline__ uint16_t buf_load2(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}

// ---------------------------------------------------------------------------
// Element type traits.  For bf16 the MFMA is v_mfma_f32_32x32x16_bf16: each
// lane carries 8 consecutive k values.  For fp32 it is
// v_mfma_f32_32x32x2_f32: one k value per lane.
//   A operand (32 x K): lane l holds row l%32, k = (l/32)*KP .. +KP
//   B operand (K x 32): lane l holds col l%32, k = (l/32)*KP .. +KP
//   C/D (32 x 32): lane l holds col l%32, rows (i/4)*8 + (l/32)*4 + i%4
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<bf16> {
  static constexpr int KP = 8;  // k values per lane per MFMA
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
};

template <>
struct Elem<float> {
  static constexpr int KP = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f32(float x) { return x; }
};

// Row (within a 32-row MFMA output block) held in accumulator slot i by the
// lane half g = lane/32.
__device__ __forceinline__ constexpr int acc_row(int i, int g) {
  return (i >> 2) * 8 + g * 4 + (i & 3);
}

// Contraction over a 32-long index that an accumulator holds in the acc_row
// order is fed to the next MFMA without reshuffling by storing the other
// operand permuted: position g*16 + i holds index acc_row(i, g).
__device__ __forceinline__ constexpr int perm32(int r) {
  return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

// Combine lane l with lane l^32.  v_permlane32_swap with both operands = x
// leaves {x of lane l%32, x of lane l%32 + 32} in every lane, so both halves
// compute the same value in the same order.
__device__ __forceinline__ float wave_xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sliding window ("Training GEM at LLM scale", section "BlockAttention":
// each token attends only to nearby tokens; the window kernel never visits
// tiles outside the window).  Query row i sees key j iff
// i - left <= j <= i + right, both inside the sample.
struct Window {
  int left, right, lq, lk;
  // every pair of rows r0..r0+31 x keys k0..k0+31 is visible
  __device__ __forceinline__ bool full(int r0, int k0) const {
    return k0 + 31 - r0 <= right && r0 + 31 - k0 <= left && k0 + 31 < lk && r0 + 31 < lq;
  }
  __device__ __forceinline__ bool allows(int r, int k) const {
    return k - r <= right && r - k <= left && k < lk && r < lq;
  }
};
// First inner-loop step of a windowed unit whose own tile starts at row r0;
// its partners start at max(0, r0 - near).
__device__ __forceinline__ int window_first_step(int r0, int near, int step_rows) {
  return max(0, r0 - near) / step_rows;
}
// A masked score in log2 units; a running max starts no lower than kNoScore
// so that a row whose first keys are all masked stays finite.
constexpr float kNoScore = -16384.0f;

// ALU-only GELU ("Training GEM at LLM scale", section "Generalized
// Dot-Product Attention (GDPA)", item on the ALU-only activation): GELU's
// tanh form 0.5 x (1 + tanh(c (x + a x^3))), c = sqrt(2/pi), a = 0.044715,
// with tanh replaced by its Taylor polynomial through order 6,
// t(u) = u - u^3/3 + 2 u^5/15; its derivative is a polynomial as well.
// Meant for the bounded scores that QK-norm gives.
constexpr float kGeluTanhC = 0.7978845608028654f;
constexpr float kGeluTanhA = 0.044715f;
__device__ __forceinline__ float gelu_poly_u(float x) { return kGeluTanhC * x * fmaf(kGeluTanhA, x * x, 1.0f); }
__device__ __forceinline__ float tanh_poly(float u) {
  const float u2 = u * u;
  return u * fmaf(u2, fmaf(u2, 2.0f / 15.0f, -1.0f / 3.0f), 1.0f);
}
__device__ __forceinline__ float gelu_poly(float x) { return 0.5f * x * (1.0f + tanh_poly(gelu_poly_u(x))); }
__device__ __forceinline__ float gelu_poly_grad(float x) {
  const float u = gelu_poly_u(x), u2 = u * u;
  const float dt = fmaf(u2, fmaf(u2, 2.0f / 3.0f, -1.0f), 1.0f);   // t'(u)
  const float du = kGeluTanhC * fmaf(3.0f * kGeluTanhA, x * x, 1.0f);  // u'(x)
  return 0.5f * (1.0f + tanh_poly(u)) + 0.5f * x * dt * du;
}

// erf-GELU, SiLU and the ALU-only GELU (GDPA activations) and their
// derivatives, fp32.
__device__ __forceinline__ float act_fwd(int act, float x) {
  if (act == kGeluPoly) return gelu_poly(x);
  if (act == kGelu) return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
  // SiLU: x * sigmoid(x)
  return x / (1.0f + __expf(-x));
}
__device__ __forceinline__ float act_grad(int act, float x) {
  if (act == kGeluPoly) return gelu_poly_grad(x);
  if (act == kGelu) {
    const float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
    const float pdf = 0.3989422804014327f * __expf(-0.5f * x * x);
    return cdf + x * pdf;
  }
  const float s = 1.0f / (1.0f + __expf(-x));
  return s * (1.0f + x * (1.0f - s));
}

// Pack 8 fp32 values into a bf16 MFMA fragment (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)x[j];
  return r;
}

}  // namespace jattn
