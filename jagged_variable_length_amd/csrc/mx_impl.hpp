// MXFP8 jagged attention for gfx950: quantisation of bf16 tensors into MXFP8
// blocks and the forward pass on v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Method: "Training GEM at LLM scale" (Meta engineering post), section
// "Mixed Ultra-Low-Precision Training", part "Low Precision Flash Attention":
// the attention products are MXFP8 block-scaled matrix products; each tensor
// is quantised once with one scale per square 32 x 32 block (a block and its
// transpose share the scale, so the same quantisation serves the products
// that read a tensor transposed); P is converted to MXFP8 inside the
// softmax, its shared exponent taken from the row maximum softmax already
// keeps.
//
// MXFP8 tensor (one of Q, K, V, dO) of a jagged [T, H, D] bf16 tensor:
//   codes    uint8 [T, H, D]        FP8 E4M3 (OCP) codes, row-major, unpadded
//   codes_t  uint8 [RB, H, D, 32]   the same codes, one 32-token block at a
//                                   time, feature-major (token fastest); the
//                                   tokens past a sample's end are zero
//   scales   uint8 [RB, H, D/32]    E8M0 exponent X + 127 of each 32 x 32 block
// RB = sum over samples of ceil(len / 32); a sample's blocks are consecutive
// and start at the row-block base kept in its sample-table entry.  gfx950's
// MFMA reads both operands K-contiguous per lane, so a product that reduces
// over tokens (P V, and in the backward P^T dO, dS^T Q, dS K) reads codes_t,
// one that reduces over features reads codes.
//
// Scale rule: X is the smallest integer with amax * 2^-X <= 448 (amax = the
// block's largest magnitude), computed from the bits of amax; elements are
// x * 2^-X rounded to E4M3, ties to even (the hardware conversion).
#pragma once
#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"
#include "ring.hpp"

namespace jattn {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// D[32x32] += A[32x64] B[64x32], FP8 E4M3 operands with E8M0 scales.  Lane l
// (g = l/32) holds row (A) / column (B) l%32: bytes 0..15 are the reduction
// elements 16g .. 16g+15 and bytes 16..31 the elements 32+16g .. 32+16g+15;
// its scale byte (X + 127) applies to the 32-element block g (elements
// 32g .. 32g+31, half of which the other lane half holds).  This assignment
// was measured on gfx950 (one lane's scale raised by one doubles exactly that
// block of its row); the MXFP8 parity tests hold the kernels to it, since any
// other pairing of elements and scales changes the products.
__device__ __forceinline__ f32x16 mx_mma(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Operand of lane half g from a row of 64 reduction elements at p: elements
// 16g .. 16g+15 and 32+16g .. 32+16g+15.
__device__ __forceinline__ i32x8 mx_frag(const char* p, int g) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p + 16 * g);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 32 + 16 * g);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// B (or A) operand of lane half g from a 32x32-block pair of accumulator
// values already packed to E4M3: w[kb][j] holds the four codes of slots
// 4j..4j+3 of block kb, i.e. (with acc_row) elements 8j + 4g' .. +3 of block
// kb for lane half g'.  Lane half g needs elements 16g .. 16g+15 of each
// block: half 0 keeps its groups j = 0, 1 and takes its partner's, half 1
// keeps j = 2, 3 and takes its partner's (two lane exchanges per block).
__device__ __forceinline__ i32x8 mx_acc_operand(const uint32_t (&w)[2][4]) {
  i32x8 r;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto x = __builtin_amdgcn_permlane32_swap(w[kb][j], w[kb][j + 2], false, false);
      r[4 * kb + 2 * j] = (int)x[0];      // elements 16g + 8j .. +3
      r[4 * kb + 2 * j + 1] = (int)x[1];  // elements 16g + 8j + 4 .. +7
    }
  return r;
}

// Smallest X in [-127, 127] with amax * 2^-X <= 448 (amax >= 0; -127 for 0).
// With amax = 1.f * 2^(e-127) (fields e, f): 448 = 1.75 * 2^8, so X = e - 135,
// plus one when the significand exceeds 1.75.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int x = (int)(u >> 23) - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return u == 0 ? -127 : max(-127, min(127, x));
}

// Four fp32 values (|v| <= 448) to four E4M3 codes, byte i = value i.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s, 64));
  return x;
}

// ---------------------------------------------------------------------------
// Quantisation.  Workgroup = one (32-row block, head); wave w = features
// 32w .. 32w+31; lane l = row l/2, features 16*(l%2) .. +15 of the block.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(2 * D) void mx_quant_kernel(MxQuantArgs a) {
  constexpr int NB = D / 32;
  __shared__ __attribute__((aligned(16))) uint8_t tile[32 * D];
  const int r = blockIdx.x / a.H, h = blockIdx.x - r * a.H;
  const int row0 = a.blocks[2 * r], nrows = a.blocks[2 * r + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane >> 1, col = wave * 32 + (lane & 1) * 16;
  const int64_t HD = (int64_t)a.H * D;
  float v[16];
  if (row < nrows) {
    const bf16* src = reinterpret_cast<const bf16*>(a.x) + (int64_t)(row0 + row) * HD + h * D + col;
    bf16x8_to_f32(reinterpret_cast<const char*>(src), v);
    bf16x8_to_f32(reinterpret_cast<const char*>(src + 8), v + 8);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  const int X = mx_scale_exp(wave_max64(m));
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = pack4_fp8(ldexpf(v[4 * j], -X), ldexpf(v[4 * j + 1], -X), ldexpf(v[4 * j + 2], -X),
                     ldexpf(v[4 * j + 3], -X));
  if (row < nrows) *reinterpret_cast<u32x4*>(a.codes + (int64_t)(row0 + row) * HD + h * D + col) = w;
  if (lane == 0) a.scales[((int64_t)r * a.H + h) * NB + wave] = (uint8_t)(X + 127);
  if (a.codes_t != nullptr) {
    // the block transposed: feature d, tokens 0..31 (rows past the sample end
    // hold the code of 0)
    *reinterpret_cast<u32x4*>(tile + row * D + col) = w;
    __syncthreads();
    const int d = threadIdx.x >> 1, t0 = (threadIdx.x & 1) * 16;
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) x |= (uint32_t)tile[(t0 + 4 * j + k) * D + d] << (8 * k);
      o[j] = x;
    }
    *reinterpret_cast<u32x4*>(a.codes_t + (((int64_t)r * a.H + h) * D + d) * 32 + t0) = o;
  }
}

// ---------------------------------------------------------------------------
// Forward.  Workgroup = 4 waves; a unit is (sample, head, 128 query rows),
// wave w owns rows 32w .. 32w+31; each step covers 64 keys (two 32-key
// blocks, the reduction length of one P V product):
//   S^T = K Q^T      A = K rows (LDS, codes), B = Q (registers, codes)
//   softmax          lane = one query row, 32 of the step's 64 keys; lazy
//                    rescale; P scaled by 2^-Xp, Xp from the step's row max
//   O^T += V^T P^T   A = V^T (LDS, codes_t), B = P after lane exchanges
// K rows and V^T come HBM -> LDS through buffer loads whose destination is
// LDS, into a ring of up to four stages filled by a producer cursor that
// runs ahead across unit boundaries (each step waits only for its own
// loads, with per-wave counts), one barrier per step.  Keys past the sample end read
// as zeros in both tiles (K rows past the descriptor end; codes_t tokens past
// the sample end are zero or past the descriptor end), so the padding
// subtraction of the bf16 kernels applies unchanged.
// ---------------------------------------------------------------------------
template <int D>
struct MxFwdShape {
  static constexpr int NW = 4, BM = 128, BN = 64;
  using KT = PadTile<D / 2, 1>;  // K rows of D bytes (as D/2 16-bit slots), pitch D + 16
  static constexpr int K_BYTES = KT::template bytes<BN>();
  static constexpr int VPITCH = 80;  // V^T rows: 64 tokens + 16 pad bytes
  static constexpr int V_SPR = 5;
  static constexpr int V_NI = (D * V_SPR + 63) / 64;
  static constexpr int V_BYTES = V_NI * 1024;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int NS_FIT = 160 * 1024 / STAGE;
  static constexpr int NS = NS_FIT >= 4 ? 4 : NS_FIT;
  static_assert(NS >= 2, "two stages at least");
  static constexpr int SMEM = NS * STAGE;
  static constexpr int KNI = KT::template ninst<BN>();  // LDS-destination loads of one step
};

// Plan records through scalar loads (wave-uniform addresses, read-only data).
typedef __attribute__((address_space(4))) const uint32_t c_u32;
__device__ __forceinline__ uint32_t sload_u32(const void* base, int64_t byte_off) {
  return ((c_u32*)base)[byte_off >> 2];
}

// The NB scale bytes of block `blk`, head h (NB = D/32 <= 4), as one word.
template <int D>
__device__ __forceinline__ uint32_t mx_scale_word(const uint8_t* scales, int64_t blk, int h, int H) {
  constexpr int NB = D / 32;
  const int64_t off = (blk * H + h) * NB;
  const uint32_t w = sload_u32(scales, off & ~int64_t(3));
  return NB == 4 ? w : (w >> (8 * (int)(off & 3)));
}
__device__ __forceinline__ int scale_byte(uint32_t word, int i) { return (int)((word >> (8 * i)) & 0xffu); }

template <typename TO, int D, int ACT>
__global__ __launch_bounds__(256, 1) void mx_fwd_kernel(MxFwdArgs a) {
  using Sh = MxFwdShape<D>;
  constexpr int BM = Sh::BM, BN = Sh::BN, ND = D / 32, NC = D / 64;
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  constexpr float kLazy = 8.0f;

  __shared__ __attribute__((aligned(1024))) char smem[Sh::SMEM];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_begin = sload1(a.worker_off, worker);
  const int u_end = sload1(a.worker_off, worker + 1);
  const int H = a.H;
  const int HD = H * D;  // bytes per token row of codes
  const int64_t BLK = (int64_t)H * D * 32;  // bytes per row block of codes_t
  constexpr int NS = Sh::NS;
  const uint32_t smem_lds = lds_addr(smem);

  RowLoader<D / 2, 1, BN, 4> kload;
  kload.init(wave, lane, HD / 2);
  static_assert(decltype(kload)::NI == Sh::KNI, "the ring's per-step counts are the loaders' instruction counts");
  // V^T loader: slot s -> feature s/5, 16-byte chunk s%5 (chunk 4 = pad);
  // chunks 0,1 from the step's first token block, 2,3 from its second
  uint32_t vvoff[(Sh::V_NI + 3) / 4];
#pragma unroll
  for (int j = 0; j < (Sh::V_NI + 3) / 4; ++j) {
    const int s = (wave + 4 * j) * 64 + lane;
    const int d = s / Sh::V_SPR, ch = s % Sh::V_SPR;
    vvoff[j] = (ch < 4 && d < D) ? (uint32_t)((ch >> 1) * BLK + d * 32 + (ch & 1) * 16) : 0x80000000u;
  }

  struct UnitInfo {
    int b, h, qt, n;
    Sample s;
    int qblk0, kblk0, nkblk;
  };
  auto fetch = [&](int u) {
    UnitInfo x;
    const i32x4 un = sload4(a.units, u);
    x.b = un[0];
    x.h = un[1];
    x.qt = un[2];
    x.n = un[3];
    x.s = sload_sample(a.samples, x.b);
    const i32x4 y = sload4(a.samples, 2 * x.b + 1);  // entries 4..7: bias0, row-block bases
    x.qblk0 = y[2];
    x.kblk0 = y[3];
    x.nkblk = (x.s.lk + 31) >> 5;
    return x;
  };
  // Q fragments (B operand) of this wave's 32 rows and their scale bytes
  auto load_q = [&](const UnitInfo& x, i32x8* qf, int* qsc) {
    const rsrc_t rq = make_rsrc(a.q.codes + ((int64_t)x.s.q0 * H + x.h) * D, (uint32_t)x.s.lq * HD);
    const int row = x.qt * BM + wave * 32 + l32;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const i32x4 lo = buf_load16(rq, (uint32_t)(row * HD + c * 64 + g * 16));
      const i32x4 hi = buf_load16(rq, (uint32_t)(row * HD + c * 64 + 32 + g * 16));
      qf[c] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    const int nqb = (x.s.lq + 31) >> 5;
    const int qb = min(x.qt * 4 + wave, nqb - 1);  // a block past the sample: any finite scale
    const uint32_t wq = mx_scale_word<D>(a.q.scales, x.qblk0 + qb, x.h, H);
#pragma unroll
    for (int c = 0; c < NC; ++c) qsc[c] = scale_byte(wq, 2 * c + g);
  };

  if (u_begin >= u_end) return;

  // ---- producer: the worker's steps in order, NS - 1 ahead of the consumer ----
  // A step moves K rows 64t .. of (sample, head) (zero past the sample end)
  // and V^T of token blocks kblk0 + 2t, + 2t + 1 (the descriptor ends with
  // the sample's last block, so a block past it reads zero).  Descriptors
  // are set up once per unit and advanced by a constant per step.
  constexpr int LOOK = NS - 1;
  constexpr int VJ = (Sh::V_NI + 3) / 4;
  const int step_ops = loads_of(Sh::KNI, wave, 4) + loads_of(Sh::V_NI, wave, 4);
  constexpr int MIN_OPS = loads_of(Sh::KNI, 3, 4) + loads_of(Sh::V_NI, 3, 4);
  constexpr int WAIT_N = (LOOK - 1) * MIN_OPS < 63 ? (LOOK - 1) * MIN_OPS : 63;
  VmLedger<LOOK, WAIT_N> ring;
  int pu = u_begin, pt = 0, pn = 0, pst = 0;
  Walker<false> w_k, w_v;
  auto start_unit = [&](const UnitInfo& x) {
    w_k.start(a.k.codes, ((int64_t)x.s.k0 * H + x.h) * D, (int64_t)x.s.lk * HD);
    const int64_t vb = (int64_t)x.kblk0 * H + x.h;
    const int64_t vend = ((int64_t)(x.kblk0 + x.nkblk - 1) * H + x.h + 1) * D * 32;
    w_v.start(a.v.codes_t, vb * D * 32, vend - vb * D * 32);
  };
  UnitInfo pinfo = fetch(u_begin);
  pn = pinfo.n;
  if (pn > 0) start_unit(pinfo);
  auto produce = [&]() {
    if (pt >= pn && pu < u_end) {
      do {
        ++pu;
        if (pu < u_end) pinfo = fetch(pu);
      } while (pu < u_end && pinfo.n == 0);
      pt = 0;
      pn = pu < u_end ? pinfo.n : 0;
      if (pn > 0) start_unit(pinfo);
    }
    if (pt < pn) {
      const uint32_t sb = smem_lds + pst * Sh::STAGE;
      kload.issue(sb, w_k.words(), wave);
      const i32x4 rvs = w_v.words();
#pragma unroll
      for (int j = 0; j < VJ; ++j) {
        const int inst = wave + 4 * j;
        if (inst < Sh::V_NI) lds_dma16(rvs, sb + Sh::K_BYTES + inst * 1024, vvoff[j]);
      }
      w_k.advance((int64_t)BN * HD);
      w_v.advance(2 * BLK);
      ++pt;
      pst = pst + 1 == NS ? 0 : pst + 1;
      ring.produced(step_ops);
    } else {
      ring.produced(0);
    }
  };

  UnitInfo cur = fetch(u_begin);
  i32x8 qf[NC];
  int qsc[NC];
  load_q(cur, qf, qsc);
  // the first unit's Q has landed before anything else is issued (see the
  // bf16 forward: later Q loads are followed by visible stores)
  wait_vmcnt<0>();
  for (int j = 0; j < LOOK; ++j) produce();
  int stage = 0;

  for (int u = u_begin; u < u_end; ++u) {
    const bool has_next = u + 1 < u_end;
    UnitInfo nxt = cur;
    if (has_next) nxt = fetch(u + 1);
    const int n = cur.n;

    f32x16 oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};
    float m_run = 0.0f, l_run = 0.0f;
    bool pad_drop = false;

    // LAST (step n-1) alone loads the next unit's Q: the loop over the other
    // steps then carries no register loads for the compiler to wait on
    auto step = [&](auto first_tag, auto last_tag, int t) {
      constexpr bool FIRST = decltype(first_tag)::value;
      constexpr bool LAST = decltype(last_tag)::value;
      ring.wait_oldest();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // step t is in LDS; every wave is done with the stage produce() refills
      __builtin_amdgcn_sched_barrier(0);
      produce();
      const char* kt = smem + stage * Sh::STAGE;
      const char* vt = kt + Sh::K_BYTES;
      // scale words of the step's two key blocks (a block past the sample: any finite scale)
      int kb_idx[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kb_idx[kb] = cur.kblk0 + min(2 * t + kb, cur.nkblk - 1);
      const uint32_t ksw0 = mx_scale_word<D>(a.k.scales, kb_idx[0], cur.h, H);
      const uint32_t ksw1 = mx_scale_word<D>(a.k.scales, kb_idx[1], cur.h, H);
      const uint32_t vsw0 = mx_scale_word<D>(a.v.scales, kb_idx[0], cur.h, H);
      const uint32_t vsw1 = mx_scale_word<D>(a.v.scales, kb_idx[1], cur.h, H);

      // ---- S^T = K Q^T: rows = 64 keys (two blocks), columns = 32 queries ----
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t ksw = kb ? ksw1 : ksw0;
        const char* krow = kt + Sh::KT::off(kb * 32 + l32, 0);
#pragma unroll
        for (int c = 0; c < NC; ++c)
          sacc[kb] = mx_mma(mx_frag(krow + c * 64, g), qf[c], sacc[kb], scale_byte(ksw, 2 * c + g), qsc[c]);
      }
      // Q is dead after the last S^T of the unit: fetch the next unit's rows
      if (LAST && has_next) load_q(nxt, qf, qsc);

      // slot (kb, i) of lane (query l32, g) holds key 64t + 32kb + acc_row(i, g)
      float p[2][16];
      int xp[2];  // E8M0 exponent of P per key block
      if constexpr (SOFTMAX) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) p[kb][i] = fmaf(sacc[kb][i], a.scale_log2, -m_run);
        // guard of the subtraction scheme (see the bf16 forward): a row whose
        // best valid score in the last step is below 0 drops the padded keys
        const int rem = cur.s.lk - t * BN;  // valid keys of this step
        if (LAST && rem < BN) {
          float vm = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) vm = kb * 32 + acc_row(i, g) < rem ? fmaxf(vm, p[kb][i]) : vm;
          vm = wave_xor32_max(vm);
          pad_drop = (FIRST ? vm : m_run + fmaxf(vm, 0.0f)) < 0.0f;
          if (pad_drop) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) p[kb][i] = kb * 32 + acc_row(i, g) < rem ? p[kb][i] : -INFINITY;
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, p[kb][i]);
        mx = wave_xor32_max(mx);
        float rel;  // largest exponent (log2) of this step's P after any rescale
        if constexpr (FIRST) {
          m_run = mx;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) p[kb][i] -= m_run;
          rel = 0.0f;
        } else {
          rel = mx;
          if (__builtin_amdgcn_ballot_w64(mx > kLazy) != 0) {
            const float delta = fmaxf(mx, 0.0f);
            const float alpha = fast_exp2(-delta);
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
            m_run += delta;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) p[kb][i] -= delta;
            rel = mx - delta;
          }
        }
        // P = 2^p <= 2^rel: the shared exponent Xp = ceil(rel) - 8 keeps every
        // P * 2^-Xp <= 256; the elements 2^(p - Xp) come straight from exp2
        const int X = max(-127, (int)ceilf(rel) - 8);
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[kb][i] = fast_exp2(p[kb][i] - (float)X);
            rs += p[kb][i];
          }
        l_run += ldexpf(rs, X);
        xp[0] = xp[1] = X;
      } else {
        // GDPA: P = act(S); each 32-key block of a row gets the scale of its
        // largest |P| (the two lane halves of the row share it)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float am = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[kb][i] = act_fwd(ACT, sacc[kb][i] * a.scale);
            am = fmaxf(am, fabsf(p[kb][i]));
          }
          xp[kb] = mx_scale_exp(wave_xor32_max(am));
#pragma unroll
          for (int i = 0; i < 16; ++i) p[kb][i] = ldexpf(p[kb][i], -xp[kb]);
        }
      }

      // ---- P to E4M3, rearranged into the B operand of lane half g ----
      uint32_t w[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[kb][j] = pack4_fp8(p[kb][4 * j], p[kb][4 * j + 1], p[kb][4 * j + 2], p[kb][4 * j + 3]);
      const i32x8 pb = mx_acc_operand(w);
      const int psc = (g ? xp[1] : xp[0]) + 127;  // lane half g carries block g's scale

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        oacc[d] = mx_mma(mx_frag(vt + (d * 32 + l32) * Sh::VPITCH, g), pb, oacc[d], scale_byte(g ? vsw1 : vsw0, d),
                         psc);
      }
      stage = stage + 1 == NS ? 0 : stage + 1;
    };
    if (n == 1) {
      step(std::true_type{}, std::true_type{}, 0);
    } else if (n > 1) {
      step(std::true_type{}, std::false_type{}, 0);
      for (int t = 1; t + 1 < n; ++t) step(std::false_type{}, std::false_type{}, t);
      step(std::false_type{}, std::true_type{}, n - 1);
    }

    // ---- epilogue ----
    if constexpr (SOFTMAX) {
      l_run = wave_xor32_sum(l_run);
      int npad = 0;
      if (n > 0 && !pad_drop) npad = n * BN - cur.s.lk;
      if (npad > 0) l_run -= (float)npad * fast_exp2(-m_run);
    }
    // buffer stores issued by every lane (rows past the sample end at an
    // out-of-range offset): the count the ring's waits rely on does not
    // depend on the data, and the stores stay in flight across later waits
    const int qrow = cur.qt * BM + wave * 32 + l32;
    const bool valid_row = qrow < cur.s.lq;
    {
      const bool has_keys = cur.s.lk > 0;
      float inv = 1.0f;
      if constexpr (SOFTMAX) inv = has_keys ? 1.0f / l_run : 0.0f;
      const rsrc_t ro = make_rsrc(reinterpret_cast<const TO*>(a.o) + ((int64_t)cur.s.q0 * H + cur.h) * D,
                                  (uint32_t)cur.s.lq * HD * (uint32_t)sizeof(TO));
      const uint32_t vrow = valid_row ? (uint32_t)(qrow * HD) * (uint32_t)sizeof(TO) : 0x80000000u;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          buf_store4<TO>(ro, vrow + (uint32_t)(d * 32 + i4 * 8 + g * 4) * (uint32_t)sizeof(TO),
                         oacc[d][i4 * 4] * inv, oacc[d][i4 * 4 + 1] * inv, oacc[d][i4 * 4 + 2] * inv,
                         oacc[d][i4 * 4 + 3] * inv);
      ring.counted(ND * 4);
      if (SOFTMAX && a.lse != nullptr) {
        const rsrc_t rl = make_rsrc(a.lse + (int64_t)cur.s.q0 * H + cur.h, (uint32_t)cur.s.lq * H * 4);
        const float lse = has_keys ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl,
                                              valid_row && g == 0 ? (uint32_t)qrow * H * 4 : 0x80000000u, 0, 0);
        ring.counted(1);
      }
    }

    if (has_next && n == 0) {
      // a unit without keys did not load the next Q (rare: wait here)
      load_q(nxt, qf, qsc);
      wait_vmcnt<0>();
    }
    cur = nxt;
  }
  // every production was acquired; only stores can still be in flight
  wait_vmcnt<0>();
}

}  // namespace jattn
