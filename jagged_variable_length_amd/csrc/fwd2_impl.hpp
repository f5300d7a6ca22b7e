// Forward kernel of jagged attention for bf16 inputs, gfx950 (dense mask).
//
// Method: "Training GEM at LLM scale" (Meta engineering post), sections
// "Jagged Sequence Flash Attention" (FlashAttention over jagged tensors; tail
// rows zero-filled, spurious exponentials subtracted instead of a -inf mask;
// persistent kernels) and "Generalized Dot-Product Attention (GDPA)"
// (activation in place of softmax).
//
// Workgroup = WQ x WK waves.  A unit is (sample, head, q-tile of 32*WQ rows);
// each K/V step covers BN = 32*WK keys; wave (wq, wk) computes its 32 query
// rows against key block wk of the step:
//     S^T = K Q^T      A = K rows (LDS), B = Q fragments (registers)
//     softmax          each lane owns one query row; lazy rescale
//     O^T += V^T P^T   A = V^T via ds_read_b64_tr_b16 from the row-major V
//                      tile, B = P taken straight from the S^T accumulator
// K, V and the bias tile travel HBM -> LDS with buffer loads whose
// destination is LDS (no registers, rows past the sample end read as zero),
// double-buffered so that step t+1 (or the next unit's first step) loads
// while step t computes; one barrier per step.  The key-split partials of
// one query group are combined through LDS at the end of a unit.
#pragma once
#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace jattn {

template <int D, int WQ, int WK, bool BIAS>
struct Fwd2Shape {
  static constexpr int NW = WQ * WK;          // waves
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int BM = 32 * WQ;          // query rows per unit
  static constexpr int BN = 32 * WK;          // keys per step
  static constexpr int ND = D / 32;
  static constexpr int NKK = D / 16;
  using KT = PadTile<D, 1>;  // K rows: pitch = 16 (mod 256) bytes, row reads conflict-free
  using VT = PadTile<D, 2>;  // V rows: pitch = 32 (mod 256) bytes, for transposed reads
  static constexpr int K_BYTES = KT::template bytes<BN>();
  static constexpr int V_BYTES = VT::template bytes<BN>();
  static constexpr int BROW = BN * 4 + 16;     // bias row: BN 4-byte slots + pad
  static constexpr int B_BYTES = BIAS ? BM * BROW : 0;
  static constexpr int STAGE = K_BYTES + V_BYTES + B_BYTES;
  static constexpr int COMB_O = (WK - 1) * WQ * 32 * D * 4;  // partial O of key halves 1..WK-1
  static constexpr int STATS = (WK - 1) * WQ * 32 * 3 * 4;   // their m, l, l_rounded
  static constexpr bool O_IN_STAGE = (WK > 1) && STAGE >= COMB_O;
  static constexpr bool S_IN_STAGE = (WK > 1) && STAGE >= COMB_O + STATS;
  static constexpr int EXTRA = (WK > 1) ? ((O_IN_STAGE ? 0 : COMB_O) + (S_IN_STAGE ? 0 : STATS)) : 0;
  static constexpr int SMEM = 2 * STAGE + EXTRA;
  static constexpr int BIAS_ROWS = BM * (BN / 64);  // 64-key bias row segments per step
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(!BIAS || (BIAS_ROWS % NW == 0 && NW % (BN / 64) == 0), "bias segments must deal evenly");
};

template <typename TO, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT>
__global__ __launch_bounds__(64 * WQ * WK, 1) void fwd2_kernel(FwdArgs a) {
  using Sh = Fwd2Shape<D, WQ, WK, BIAS>;
  constexpr int BM = Sh::BM, BN = Sh::BN, ND = Sh::ND, NKK = Sh::NKK, NW = Sh::NW;
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  constexpr float kLazy = 8.0f;  // rescale only when a row max grows by > 2^8

  __shared__ __attribute__((aligned(1024))) char smem[Sh::SMEM];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int wq = wave % WQ, wk = wave / WQ;
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_begin = uniform(a.worker_off[worker]);
  const int u_end = uniform(a.worker_off[worker + 1]);
  const int HD = a.H * D;

  auto stage_k = [&](int s) { return smem + s * Sh::STAGE; };
  auto stage_v = [&](int s) { return smem + s * Sh::STAGE + Sh::K_BYTES; };
  auto stage_b = [&](int s) { return smem + s * Sh::STAGE + Sh::K_BYTES + Sh::V_BYTES; };
  const uint32_t smem_lds = lds_addr(smem);

  RowLoader<D, 1, BN, NW> kload;
  RowLoader<D, 2, BN, NW> vload;
  kload.init(wave, lane, HD);
  vload.init(wave, lane, HD);

  struct UnitInfo {
    int b, h, qt, n;
    Sample s;
    i32x4 rk, rv, rb;  // descriptors at row 0 of this (sample, head)
  };
  auto fetch = [&](int u) {
    UnitInfo x;
    const i32x4 un = load_unit(a.units, u);
    x.b = un[0];
    x.h = un[1];
    x.qt = un[2];
    x.n = un[3];
    x.s = load_sample(a.samples, x.b);
    const int64_t kvo = ((int64_t)x.s.k0 * a.H + x.h) * D;
    x.rk = rsrc_words(reinterpret_cast<const bf16*>(a.k) + kvo, 0);
    x.rv = rsrc_words(reinterpret_cast<const bf16*>(a.v) + kvo, 0);
    if constexpr (BIAS)
      x.rb = rsrc_words(reinterpret_cast<const bf16*>(a.bias) + x.s.bias0 + (int64_t)x.h * x.s.lq * x.s.lk, 0);
    return x;
  };
  // issue the HBM -> LDS loads of step t of unit x into stage st: the K and V
  // descriptors start at the step's first key row and end at the sample end
  auto issue_step = [&](const UnitInfo& x, int t, int st) {
    const uint32_t sb = smem_lds + st * Sh::STAGE;
    const int64_t row0 = (int64_t)t * BN;
    const int64_t rec = (int64_t)(x.s.lk - t * BN) * HD * 2;
    kload.issue(sb, rsrc_at(x.rk, row0 * HD * 2, rec), wave);
    vload.issue(sb + Sh::K_BYTES, rsrc_at(x.rv, row0 * HD * 2, rec), wave);
    if constexpr (BIAS) {
      // one 64-key segment of one query row per load, lane l -> key l; the
      // descriptor covers exactly the valid part of the segment.  A wave
      // keeps one segment column and walks down the rows.
      constexpr int SEGS = BN / 64, RSTEP = NW / SEGS;
      const int cc = wave % SEGS, c0 = t * BN + cc * 64;
      const int nk = max(min(x.s.lk - c0, 64), 0) * 2;
      int qr = x.qt * BM + wave / SEGS;
      i32x4 rb = rsrc_at(x.rb, ((int64_t)qr * x.s.lk + c0) * 2, 0);
      uint32_t m0 = sb + Sh::K_BYTES + Sh::V_BYTES + (wave / SEGS) * Sh::BROW + cc * 256;
      const int64_t row_bytes = (int64_t)RSTEP * x.s.lk * 2;
#pragma unroll
      for (int j = 0; j < Sh::BIAS_ROWS / NW; ++j) {
        rb[2] = qr < x.s.lq ? nk : 0;
        lds_dma2(rb, m0, lane * 2);
        rb = rsrc_at(rb, row_bytes, 0);
        m0 += RSTEP * Sh::BROW;
        qr += RSTEP;
      }
    }
  };
  // Q fragments (B operand) of this wave's 32 rows, straight into registers
  auto load_q = [&](const UnitInfo& x, bf16x8* qf) {
    const rsrc_t rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + ((int64_t)x.s.q0 * a.H + x.h) * D,
                                (uint32_t)x.s.lq * HD * 2);
    const int row = x.qt * BM + wq * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(row * HD + kk * 16 + g * 8) * 2));
  };

  if (u_begin >= u_end) return;
  UnitInfo cur = fetch(u_begin);
  bf16x8 qf[NKK];
  load_q(cur, qf);
  int stage = 0;
  if (cur.n > 0) issue_step(cur, 0, 0);

  for (int u = u_begin; u < u_end; ++u) {
    const bool has_next = u + 1 < u_end;
    UnitInfo nxt = cur;
    if (has_next) nxt = fetch(u + 1);
    const int n = cur.n;

    f32x16 oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};
    float m_run = 0.0f, l_run = 0.0f, lr_run = 0.0f;

    for (int t = 0; t < n; ++t) {
      wait_vmcnt0();
      __syncthreads();  // step t is in LDS; every wave is done with step t-1
      if (t + 1 < n) {
        issue_step(cur, t + 1, stage ^ 1);
      } else if (has_next && nxt.n > 0) {
        issue_step(nxt, 0, stage ^ 1);
      }
      const char* kt = stage_k(stage);
      const char* vt = stage_v(stage);
      const int kb = wk * 32;  // this wave's key block inside the step

      f32x16 sacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) sacc = Elem<bf16>::mma(rows_frag<D, 1>(kt, kb + l32, kk, g), qf[kk], sacc);
      // Q is dead after the last S^T of the unit: fetch the next unit's rows
      if (t + 1 == n && has_next) load_q(nxt, qf);

      float p[16];
      if constexpr (BIAS) {
        const char* bt = stage_b(stage);
        const int r = wq * 32 + l32;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int c = kb + a4 * 8 + g * 4;  // 4 consecutive keys
          const u32x4 w = *reinterpret_cast<const u32x4*>(bt + r * Sh::BROW + c * 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) p[a4 * 4 + j] = __uint_as_float(w[j] << 16);
        }
      }
      bf16x8 pf[2], pl[2];
      if constexpr (SOFTMAX) {
        // scores in log2 units relative to the running max: x - m
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float c = BIAS ? fmaf(p[i], kLog2e, -m_run) : -m_run;
          p[i] = fmaf(sacc[i], a.scale_log2, c);
          mx = fmaxf(mx, p[i]);
        }
        mx = wave_xor32_max(mx);
        if (t == 0) {
          // first step: the running max starts at this step's max (m_run was 0)
          m_run = mx;
#pragma unroll
          for (int i = 0; i < 16; ++i) p[i] -= mx;
        } else if (__builtin_amdgcn_ballot_w64(mx > kLazy) != 0) {
          const float delta = fmaxf(mx, 0.0f);
          const float alpha = fast_exp2(-delta);
          l_run *= alpha;
          lr_run *= alpha;
#pragma unroll
          for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
          m_run += delta;
#pragma unroll
          for (int i = 0; i < 16; ++i) p[i] -= delta;
        }
        float rs = 0.0f, rsr = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = fast_exp2(p[i]);
          rs += p[i];
        }
        // the PV MFMA sees P rounded to bf16; the output is normalised by the
        // sum of exactly those values (v_dot2_f32_bf16 against ones)
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          pf[st] = pack8(&p[st * 8]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            rsr = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[st][2 * j], pf[st][2 * j + 1]}, ones, rsr, false);
        }
        l_run += rs;
        lr_run += rsr;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = BIAS ? p[i] + sacc[i] * a.scale : sacc[i] * a.scale;
          p[i] = act_fwd(ACT, x);
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          pf[st] = pack8(&p[st * 8]);
          if constexpr (SPLIT) {
            float r8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) r8[j] = p[st * 8 + j] - (float)pf[st][j];
            pl[st] = pack8(r8);
          }
        }
      }

#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const bf16x8 vf = trans_frag<D, 2>(vt, wk, st, d * 32, lane);
          oacc[d] = Elem<bf16>::mma(vf, pf[st], oacc[d]);
          // split operands matter for the activation path only: softmax
          // already normalises by the sum of the rounded P
          if constexpr (SPLIT && !SOFTMAX) oacc[d] = Elem<bf16>::mma(vf, pl[st], oacc[d]);
        }
      }
      stage ^= 1;
    }

    // ---- epilogue ----
    if constexpr (SOFTMAX) {
      // keys past the sample end entered the last step as zeros
      int npad = 0;
      if (n > 0) npad = 32 - min(max(cur.s.lk - ((n - 1) * BN + wk * 32), 0), 32);
      const float pad_e = fast_exp2(-m_run);
      l_run = wave_xor32_sum(l_run) - (float)npad * pad_e;
      lr_run = wave_xor32_sum(lr_run) - (float)npad * (float)(bf16)pad_e;
      if (cur.s.lk <= wk * 32) {
        // this wave's key block lies wholly past the sample end: it holds no
        // term of the row (its O is zero since those V rows read as zero)
        m_run = -INFINITY;
        l_run = 0.0f;
        lr_run = 0.0f;
      }
    }
    const int qrow = cur.qt * BM + wq * 32 + l32;
    TO* orow = reinterpret_cast<TO*>(a.o) + ((int64_t)(cur.s.q0 + qrow) * a.H + cur.h) * D;
    const bool valid_row = qrow < cur.s.lq;
    const bool has_keys = cur.s.lk > 0;

    if constexpr (WK > 1) {
      // stage that held the last step is free once every wave passes this barrier
      __syncthreads();
      char* free_stage = smem + (stage ^ 1) * Sh::STAGE;
      float* po = reinterpret_cast<float*>(Sh::O_IN_STAGE ? free_stage : smem + 2 * Sh::STAGE);
      float* ps = reinterpret_cast<float*>(Sh::S_IN_STAGE ? free_stage + Sh::COMB_O
                                                          : smem + 2 * Sh::STAGE + (Sh::O_IN_STAGE ? 0 : Sh::COMB_O));
      // element (row r of the 32-column block d, query l32) of a partial sits
      // at [slot][d*32 + r][l32]; lane-dependent parts go into one base
      const int lane_off = g * 4 * 32 + l32;
      if (wk > 0) {
        const int slot = (wk - 1) * WQ + wq;
        float* pw = po + slot * D * 32 + lane_off;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) pw[(d * 32 + (i >> 2) * 8 + (i & 3)) * 32] = oacc[d][i];
        if (g == 0) {
          ps[(slot * 3 + 0) * 32 + l32] = m_run;
          ps[(slot * 3 + 1) * 32 + l32] = l_run;
          ps[(slot * 3 + 2) * 32 + l32] = lr_run;
        }
      }
      __syncthreads();
      if (wk == 0) {
        float mall = m_run;
        if constexpr (SOFTMAX) {
#pragma unroll
          for (int w2 = 1; w2 < WK; ++w2) mall = fmaxf(mall, ps[(((w2 - 1) * WQ + wq) * 3) * 32 + l32]);
        }
        const float f0 = SOFTMAX ? (has_keys ? fast_exp2(m_run - mall) : 0.0f) : 1.0f;
        float lall = l_run * f0, lrall = lr_run * f0;
#pragma unroll
        for (int d = 0; d < ND; ++d) oacc[d] *= f0;
#pragma unroll
        for (int w2 = 1; w2 < WK; ++w2) {
          const int slot = (w2 - 1) * WQ + wq;
          float f = 1.0f;
          if constexpr (SOFTMAX) {
            f = has_keys ? fast_exp2(ps[(slot * 3) * 32 + l32] - mall) : 0.0f;
            lall += ps[(slot * 3 + 1) * 32 + l32] * f;
            lrall += ps[(slot * 3 + 2) * 32 + l32] * f;
          }
          const float* pr = po + slot * D * 32 + lane_off;
#pragma unroll
          for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[d][i] += f * pr[(d * 32 + (i >> 2) * 8 + (i & 3)) * 32];
        }
        m_run = mall;
        l_run = lall;
        lr_run = lrall;
      }
    }

    if (wk == 0 && valid_row) {
      float inv = 1.0f;
      if constexpr (SOFTMAX) inv = has_keys ? 1.0f / lr_run : 0.0f;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          store4<TO>(orow + d * 32 + i4 * 8 + g * 4, oacc[d][i4 * 4] * inv, oacc[d][i4 * 4 + 1] * inv,
                     oacc[d][i4 * 4 + 2] * inv, oacc[d][i4 * 4 + 3] * inv);
      if (SOFTMAX && a.lse != nullptr && g == 0)
        a.lse[((int64_t)cur.s.q0 + qrow) * a.H + cur.h] = has_keys ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    }

    if (has_next) {
      if (n == 0) load_q(nxt, qf);  // a unit without keys issued no prefetch
      if (n == 0 && nxt.n > 0) {
        wait_vmcnt0();
        __syncthreads();  // nobody reads LDS in a keyless unit, but keep stage order
        issue_step(nxt, 0, stage);
      }
    }
    cur = nxt;
  }
}

}  // namespace jattn
