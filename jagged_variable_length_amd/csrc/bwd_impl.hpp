// Backward kernels of jagged attention (dense mask), gfx950.
//
// Method: "Training GEM at LLM scale" (Meta engineering post), section
// "Jagged Sequence Flash Attention", item "Backward parallelization": dQ is
// computed in its own pass, separate from dK/dV, so that no output is
// accumulated with atomic adds.  Here every output element has exactly one
// writer, which also makes results bitwise reproducible.
//
//   Di kernel   : Di = rowsum(dO * O)                          (softmax only)
//   dQ kernel   : unit = (sample, head, q-tile); loop over K/V tiles
//                 S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - Di)
//                 (or act'(S^T) dP^T for GDPA), dQ^T += K^T dS^T
//   dK/dV kernel: unit = (sample, head, kv-tile); loop over Q tiles
//                 S = Q K^T, dP = dO V^T, dS as above,
//                 dV^T += dO^T P, dK^T += Q^T dS, dBias = dS
// In the dQ kernel a lane owns one query row (row statistics in-lane); in the
// dK/dV kernel a lane owns one key row.  Operands that are contracted along
// the row index (K for dQ; Q and dO for dK/dV) are staged transposed in LDS
// with the 32-block permutation that matches the MFMA accumulator layout.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"

namespace jattn {

// ---------------------------------------------------------------------------
// Di = sum_d dO * O   (one 16-byte chunk per lane, reduced across the row)
// ---------------------------------------------------------------------------
template <typename TO, typename TI, int D>
__global__ __launch_bounds__(kThreads) void di_kernel(DiArgs a) {
  constexpr int CE = 16 / (int)sizeof(TI);  // dO elements per chunk
  constexpr int LPR = D / CE;               // lanes per row
  constexpr int RPB = kThreads / LPR;       // rows per block
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int c = (tid % LPR) * CE;
  float acc = 0.0f;
  if (row < a.rows) {
    const TI* dp = reinterpret_cast<const TI*>(a.dout) + row * D + c;
    const TO* op = reinterpret_cast<const TO*>(a.o) + row * D + c;
#pragma unroll
    for (int e = 0; e < CE; ++e) acc += Elem<TI>::to_f32(dp[e]) * (float)op[e];
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < a.rows && (tid % LPR) == 0) {
    a.di[row] = acc;
    if (a.lse2 != nullptr) a.lse2[row] = a.lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ kernel.  Same tiling as the forward: 4 waves, 32 query rows per wave,
// WQ x WK waves (WK > 1 splits the key tiles of one 32-row query group).
// ---------------------------------------------------------------------------
template <typename TI, typename TG, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(BwdArgs a) {
  using E = Elem<TI>;
  using Sh = FwdShape<TI, D, WQ, WK>;
  constexpr int KP = Sh::KP, KK = Sh::KK, NKK = Sh::NKK, BM = Sh::BM, NBW = Sh::NBW;
  constexpr int BN = Sh::BN, ND = Sh::ND, CE = Sh::CE, CPR = Sh::CPR, CPT = Sh::CPT;
  constexpr int GRP = Sh::GRP, KPITCH = Sh::KPITCH, VPITCH = Sh::VPITCH, BPITCH = Sh::BPITCH;
  constexpr int BPT = Sh::BPT;
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  constexpr int SZ = (int)sizeof(TI);

  constexpr int kStageBytes = SZ * (2 * BN * KPITCH + D * VPITCH + (BIAS ? BM * BPITCH : 0));
  constexpr int kCombineBytes = (WK > 1) ? (int)sizeof(float) * WK * D * 32 : 0;
  constexpr int kSmem = kStageBytes > kCombineBytes ? kStageBytes : kCombineBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  TI* Ks = reinterpret_cast<TI*>(smem);  // K row-major   (A of S^T)
  TI* Vs = Ks + BN * KPITCH;             // V row-major   (A of dP^T)
  TI* Kt = Vs + BN * KPITCH;             // K transposed  (A of dQ^T)
  TI* Bs = Kt + D * VPITCH;              // bias tile [BM][BN]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wq = wave % WQ, wk = wave / WQ;
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_end = uniform(a.worker_off[worker + 1]);
  const int HD = a.H * D;
  const int sc = tid % CPR;
  const int sr0 = (tid / CPR) * CPT;
  const int bc = tid % BN;
  const int br0 = tid / BN;

  for (int u = uniform(a.worker_off[worker]); u < u_end; ++u) {
    const i32x4 unit = load_unit(a.units, u);
    const int b = unit[0], h = unit[1], qt = unit[2], ntiles = unit[3];
    const Sample s = load_sample(a.samples, b);
    const int qrow = qt * BM + wq * 32 + l32;

    const int64_t qoff = ((int64_t)s.q0 * a.H + h) * D;
    const rsrc_t rq = make_rsrc(reinterpret_cast<const TI*>(a.q) + qoff, (uint32_t)s.lq * HD * SZ);
    const rsrc_t rdo = make_rsrc(reinterpret_cast<const TI*>(a.dout) + qoff, (uint32_t)s.lq * HD * SZ);
    typename E::frag qf[NKK], dof[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint32_t voff = (uint32_t)(qrow * HD + kk * KK + g * KP) * SZ;
      if constexpr (KP == 8) {
        qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, voff));
        dof[kk] = __builtin_bit_cast(bf16x8, buf_load16(rdo, voff));
      } else {
        qf[kk] = __uint_as_float(buf_load4(rq, voff));
        dof[kk] = __uint_as_float(buf_load4(rdo, voff));
      }
    }
    float lse2 = 0.0f, di = 0.0f;  // zero for tail rows keeps them finite
    if constexpr (SOFTMAX) {
      if (qrow < s.lq) {
        const int64_t r = ((int64_t)s.q0 + qrow) * a.H + h;
        lse2 = a.lse[r] * kLog2e;
        di = a.di[r];
      }
    }

    const int64_t koff = ((int64_t)s.k0 * a.H + h) * D;
    const rsrc_t rk = make_rsrc(reinterpret_cast<const TI*>(a.k) + koff, (uint32_t)s.lk * HD * SZ);
    const rsrc_t rv = make_rsrc(reinterpret_cast<const TI*>(a.v) + koff, (uint32_t)s.lk * HD * SZ);
    rsrc_t rb = rk;
    if constexpr (BIAS) {
      const TI* bb = reinterpret_cast<const TI*>(a.bias) + s.bias0 + (int64_t)h * s.lq * s.lk;
      rb = make_rsrc(bb, (uint32_t)s.lq * s.lk * SZ);
    }

    f32x16 dqacc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) dqacc[i] = f32x16{};

    i32x4 kreg[CPT], vreg[CPT];
    uint32_t breg[BIAS ? BPT : 1];
    auto issue_loads = [&](int t) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const uint32_t voff = (uint32_t)((t * BN + sr0 + j) * HD + sc * CE) * SZ;
        kreg[j] = buf_load16(rk, voff);
        vreg[j] = buf_load16(rv, voff);
      }
      if constexpr (BIAS) {
        // rows qt*BM + br0 + i*(256/BN) of column t*BN + bc; a column past
        // the sample end is pushed out of the buffer range (reads zero)
        const int kv = t * BN + bc;
        const uint32_t step = (uint32_t)(kThreads / BN) * s.lk * SZ;
        uint32_t voff = (uint32_t)((qt * BM + br0) * s.lk + kv) * SZ;
        voff = (kv < s.lk) ? voff : 0x80000000u;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          if constexpr (SZ == 2)
            breg[i] = buf_load2(rb, voff + i * step);
          else
            breg[i] = buf_load4(rb, voff + i * step);
        }
      }
    };
    auto stage_to_lds = [&]() {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        *reinterpret_cast<i32x4*>(&Ks[(sr0 + j) * KPITCH + sc * CE]) = kreg[j];
        *reinterpret_cast<i32x4*>(&Vs[(sr0 + j) * KPITCH + sc * CE]) = vreg[j];
      }
#pragma unroll
      for (int gq = 0; gq < CPT / GRP; ++gq) {
        const int r = sr0 + gq * GRP;
        const int pr = (r & ~31) + perm32(r & 31);
#pragma unroll
        for (int e = 0; e < CE; ++e)
          TGroup<TI, GRP>::write(&Kt[(sc * CE + e) * VPITCH + pr], &kreg[gq * GRP], e);
      }
      if constexpr (BIAS) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          const int r = br0 + i * (kThreads / BN);
          if constexpr (SZ == 2)
            reinterpret_cast<uint16_t*>(Bs)[r * BPITCH + bc] = (uint16_t)breg[i];
          else
            reinterpret_cast<uint32_t*>(Bs)[r * BPITCH + bc] = breg[i];
        }
      }
    };

    if (ntiles > 0) issue_loads(0);
    for (int t = 0; t < ntiles; ++t) {
      __syncthreads();
      stage_to_lds();
      __syncthreads();
      if (t + 1 < ntiles) issue_loads(t + 1);
      const bool last = (t == ntiles - 1);

      f32x16 sacc[NBW], dpacc[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int kb = (wk * NBW + nb) * 32;
        sacc[nb] = f32x16{};
        dpacc[nb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int off = (kb + l32) * KPITCH + kk * KK + g * KP;
          typename E::frag kf, vf;
          if constexpr (KP == 8) {
            kf = *reinterpret_cast<const bf16x8*>(&Ks[off]);
            vf = *reinterpret_cast<const bf16x8*>(&Vs[off]);
          } else {
            kf = Ks[off];
            vf = Vs[off];
          }
          sacc[nb] = E::mma(kf, qf[kk], sacc[nb]);
          dpacc[nb] = E::mma(vf, dof[kk], dpacc[nb]);
        }
      }

      float ds[NBW][16];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kvl = (wk * NBW + nb) * 32 + acc_row(i, g);
          float bv = 0.0f;
          if constexpr (BIAS) bv = E::to_f32(Bs[(wq * 32 + l32) * BPITCH + kvl]);
          float d;
          if constexpr (SOFTMAX) {
            const float p = exp2f(sacc[nb][i] * a.scale_log2 + bv * kLog2e - lse2);
            d = p * (dpacc[nb][i] - di);
          } else {
            d = act_grad(ACT, sacc[nb][i] * a.scale + bv) * dpacc[nb][i];
          }
          // keys past the sample end: K is zero there, but keep dS finite
          if (last && t * BN + kvl >= s.lk) d = 0.0f;
          ds[nb][i] = d;
        }
      }

#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int kb = (wk * NBW + nb) * 32;
#pragma unroll
        for (int st = 0; st < 16 / KP; ++st) {
          typename E::frag hf, lf;
          if constexpr (KP == 8) {
            hf = pack8(&ds[nb][st * 8]);
            if constexpr (SPLIT) {
              float r[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) r[j] = ds[nb][st * 8 + j] - (float)hf[j];
              lf = pack8(r);
            }
          } else {
            hf = ds[nb][st];
          }
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const TI* src = &Kt[(d * 32 + l32) * VPITCH + kb + g * 16 + st * KP];
            typename E::frag af;
            if constexpr (KP == 8)
              af = *reinterpret_cast<const bf16x8*>(src);
            else
              af = *src;
            dqacc[d] = E::mma(af, hf, dqacc[d]);
            if constexpr (SPLIT && KP == 8) dqacc[d] = E::mma(af, lf, dqacc[d]);
          }
        }
      }
    }

    TG* gbase = reinterpret_cast<TG*>(a.dq) + ((int64_t)s.q0 * a.H + h) * D;
    if constexpr (WK == 1) {
      if (qrow < s.lq) {
        TG* grow = gbase + (int64_t)qrow * HD;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            store4<TG>(grow + d * 32 + i4 * 8 + g * 4, dqacc[d][i4 * 4 + 0] * a.scale,
                       dqacc[d][i4 * 4 + 1] * a.scale, dqacc[d][i4 * 4 + 2] * a.scale,
                       dqacc[d][i4 * 4 + 3] * a.scale);
      }
    } else {
      float* part = reinterpret_cast<float*>(smem);  // [WK][D][32]
      __syncthreads();
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) part[(wk * D + d * 32 + acc_row(i, g)) * 32 + l32] = dqacc[d][i];
      __syncthreads();
      constexpr int DC = D / WK;
      const int row = qt * BM + l32;
      if (row < s.lq) {
        TG* grow = gbase + (int64_t)row * HD;
#pragma unroll
        for (int c4 = g * 4; c4 < DC; c4 += 8) {
          float r[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = wave * DC + c4 + j;
            float acc = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < WK; ++w2) acc += part[(w2 * D + col) * 32 + l32];
            r[j] = acc * a.scale;
          }
          store4<TG>(grow + wave * DC + c4, r[0], r[1], r[2], r[3]);
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel.  A unit owns KT = 32*WKV key rows; each step consumes
// QS = 32*WKQ query rows (WKV * WKQ = 4 waves).  Wave (wv, wqs) handles key
// rows wv*32.. of the unit and query rows wqs*32.. of each step.
// ---------------------------------------------------------------------------
template <typename TI, int D, int WKV>
struct DkdvShape {
  static constexpr int KP = Elem<TI>::KP;
  static constexpr int KK = 2 * KP;
  static constexpr int NKK = D / KK;
  static constexpr int WKQ = 4 / WKV;
  static constexpr int KT = 32 * WKV;  // key rows per unit
  static constexpr int QS = 32 * WKQ;  // query rows per step
  static constexpr int ND = D / 32;
  static constexpr int CE = 16 / (int)sizeof(TI);
  static constexpr int CPR = D / CE;
  static constexpr int NCH = QS * CPR;              // Q (and dO) chunks per step
  static constexpr int CPT = NCH >= kThreads ? NCH / kThreads : 1;  // chunks per staging thread
  static constexpr int NSTG = NCH / CPT;            // threads that stage Q/dO
  static constexpr int GRP = CPT < 4 ? CPT : 4;
  static constexpr int QPITCH = D + CE;   // Qs / dOs row pitch
  static constexpr int TPITCH = QS + CE;  // Qt / dOt row pitch
  static constexpr int BPITCH = KT + 4;   // bias tile [QS][KT]
  static constexpr int BPT = QS * KT / kThreads;
  static_assert(NCH % CPT == 0 && NSTG <= kThreads, "tile/threads mismatch");
  static_assert(kThreads % KT == 0, "bias staging assumes KT | 256");
};

// DBIAS: 0 = no dBias, 1 = bf16 dBias, 2 = fp32 dBias
template <typename TI, typename TG, int D, int WKV, int ACT, bool BIAS, int DBIAS, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdArgs a) {
  using E = Elem<TI>;
  using Sh = DkdvShape<TI, D, WKV>;
  constexpr int KP = Sh::KP, KK = Sh::KK, NKK = Sh::NKK, WKQ = Sh::WKQ, KT = Sh::KT, QS = Sh::QS;
  constexpr int ND = Sh::ND, CE = Sh::CE, CPR = Sh::CPR, CPT = Sh::CPT, GRP = Sh::GRP;
  constexpr int QPITCH = Sh::QPITCH, TPITCH = Sh::TPITCH, BPITCH = Sh::BPITCH, BPT = Sh::BPT;
  constexpr int NSTG = Sh::NSTG;
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  constexpr int SZ = (int)sizeof(TI);

  constexpr int kStageBytes = SZ * (2 * QS * QPITCH + 2 * D * TPITCH + (BIAS ? QS * BPITCH : 0)) +
                              (int)sizeof(float) * 2 * QS;
  constexpr int kCombineBytes = (WKQ > 1) ? (int)sizeof(float) * 4 * 32 * (D + 1) : 0;
  constexpr int kSmem = kStageBytes > kCombineBytes ? kStageBytes : kCombineBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  TI* Qs = reinterpret_cast<TI*>(smem);  // Q rows        (A of S)
  TI* Os = Qs + QS * QPITCH;             // dO rows       (A of dP)
  TI* Qt = Os + QS * QPITCH;             // Q transposed  (A of dK^T)
  TI* Ot = Qt + D * TPITCH;              // dO transposed (A of dV^T)
  TI* Bs = Ot + D * TPITCH;              // bias tile
  float* L2s = reinterpret_cast<float*>(Bs + (BIAS ? QS * BPITCH : 0));  // LSE * log2e
  float* Dis = L2s + QS;                                                  // Di

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wv = wave % WKV, wqs = wave / WKV;
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_end = uniform(a.worker_off[worker + 1]);
  const int HD = a.H * D;
  const int sc = tid % CPR;
  const int sr0 = (tid / CPR) * CPT;
  const int bc = tid % KT;
  const int br0 = tid / KT;

  for (int u = uniform(a.worker_off[worker]); u < u_end; ++u) {
    const i32x4 unit = load_unit(a.units, u);
    const int b = unit[0], h = unit[1], kt = unit[2], nsteps = unit[3];
    const Sample s = load_sample(a.samples, b);
    const int krow = kt * KT + wv * 32 + l32;  // this lane's key row in the sample

    const int64_t koff = ((int64_t)s.k0 * a.H + h) * D;
    const rsrc_t rk = make_rsrc(reinterpret_cast<const TI*>(a.k) + koff, (uint32_t)s.lk * HD * SZ);
    const rsrc_t rv = make_rsrc(reinterpret_cast<const TI*>(a.v) + koff, (uint32_t)s.lk * HD * SZ);
    typename E::frag kf[NKK], vf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint32_t voff = (uint32_t)(krow * HD + kk * KK + g * KP) * SZ;
      if constexpr (KP == 8) {
        kf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rk, voff));
        vf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rv, voff));
      } else {
        kf[kk] = __uint_as_float(buf_load4(rk, voff));
        vf[kk] = __uint_as_float(buf_load4(rv, voff));
      }
    }

    const int64_t qoff = ((int64_t)s.q0 * a.H + h) * D;
    const rsrc_t rq = make_rsrc(reinterpret_cast<const TI*>(a.q) + qoff, (uint32_t)s.lq * HD * SZ);
    const rsrc_t rdo = make_rsrc(reinterpret_cast<const TI*>(a.dout) + qoff, (uint32_t)s.lq * HD * SZ);
    rsrc_t rb = rq;
    const int64_t bias_hb = s.bias0 + (int64_t)h * s.lq * s.lk;
    if constexpr (BIAS) rb = make_rsrc(reinterpret_cast<const TI*>(a.bias) + bias_hb, (uint32_t)s.lq * s.lk * SZ);

    f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dkacc[i] = f32x16{};
      dvacc[i] = f32x16{};
    }

    i32x4 qreg[CPT], oreg[CPT];
    uint32_t breg[BIAS ? BPT : 1];
    float lreg = 0.0f, dreg = 0.0f;
    auto issue_loads = [&](int t) {
      if (NSTG == kThreads || tid < NSTG) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const uint32_t voff = (uint32_t)((t * QS + sr0 + j) * HD + sc * CE) * SZ;
          qreg[j] = buf_load16(rq, voff);
          oreg[j] = buf_load16(rdo, voff);
        }
      }
      if constexpr (SOFTMAX) {
        if (tid < QS) {
          const int qr = t * QS + tid;
          const int64_t r = ((int64_t)s.q0 + qr) * a.H + h;
          lreg = (qr < s.lq) ? a.lse[r] * kLog2e : 0.0f;
          dreg = (qr < s.lq) ? a.di[r] : 0.0f;
        }
      }
      if constexpr (BIAS) {
        const int kv = kt * KT + bc;
        const uint32_t step = (uint32_t)(kThreads / KT) * s.lk * SZ;
        uint32_t voff = (uint32_t)((t * QS + br0) * s.lk + kv) * SZ;
        voff = (kv < s.lk) ? voff : 0x80000000u;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          if constexpr (SZ == 2)
            breg[i] = buf_load2(rb, voff + i * step);
          else
            breg[i] = buf_load4(rb, voff + i * step);
        }
      }
    };
    auto stage_to_lds = [&]() {
      if (NSTG == kThreads || tid < NSTG) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          *reinterpret_cast<i32x4*>(&Qs[(sr0 + j) * QPITCH + sc * CE]) = qreg[j];
          *reinterpret_cast<i32x4*>(&Os[(sr0 + j) * QPITCH + sc * CE]) = oreg[j];
        }
#pragma unroll
        for (int gq = 0; gq < CPT / GRP; ++gq) {
          const int r = sr0 + gq * GRP;
          const int pr = (r & ~31) + perm32(r & 31);
#pragma unroll
          for (int e = 0; e < CE; ++e) {
            TGroup<TI, GRP>::write(&Qt[(sc * CE + e) * TPITCH + pr], &qreg[gq * GRP], e);
            TGroup<TI, GRP>::write(&Ot[(sc * CE + e) * TPITCH + pr], &oreg[gq * GRP], e);
          }
        }
      }
      if constexpr (SOFTMAX) {
        if (tid < QS) {
          L2s[tid] = lreg;
          Dis[tid] = dreg;
        }
      }
      if constexpr (BIAS) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          const int r = br0 + i * (kThreads / KT);
          if constexpr (SZ == 2)
            reinterpret_cast<uint16_t*>(Bs)[r * BPITCH + bc] = (uint16_t)breg[i];
          else
            reinterpret_cast<uint32_t*>(Bs)[r * BPITCH + bc] = breg[i];
        }
      }
    };

    const int kvl = wv * 32 + l32;  // key row within the unit tile
    if (nsteps > 0) issue_loads(0);
    for (int t = 0; t < nsteps; ++t) {
      __syncthreads();
      stage_to_lds();
      __syncthreads();
      if (t + 1 < nsteps) issue_loads(t + 1);

      // S = Q K^T and dP = dO V^T for this wave's 32 queries x 32 keys
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int off = (wqs * 32 + l32) * QPITCH + kk * KK + g * KP;
        typename E::frag qa, oa;
        if constexpr (KP == 8) {
          qa = *reinterpret_cast<const bf16x8*>(&Qs[off]);
          oa = *reinterpret_cast<const bf16x8*>(&Os[off]);
        } else {
          qa = Qs[off];
          oa = Os[off];
        }
        sacc = E::mma(qa, kf[kk], sacc);
        dpacc = E::mma(oa, vf[kk], dpacc);
      }

      float p[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ql = wqs * 32 + acc_row(i, g);  // query row within the step
        float bv = 0.0f;
        if constexpr (BIAS) bv = E::to_f32(Bs[ql * BPITCH + kvl]);
        if constexpr (SOFTMAX) {
          p[i] = exp2f(sacc[i] * a.scale_log2 + bv * kLog2e - L2s[ql]);
          ds[i] = p[i] * (dpacc[i] - Dis[ql]);
        } else {
          const float x = sacc[i] * a.scale + bv;
          p[i] = act_fwd(ACT, x);
          ds[i] = act_grad(ACT, x) * dpacc[i];
        }
      }
      if constexpr (DBIAS) {
        const int kv = kt * KT + kvl;
        if (kv < s.lk) {
          typedef typename std::conditional<DBIAS == 2, float, bf16>::type TB;
          TB* db = reinterpret_cast<TB*>(a.dbias) + bias_hb + kv;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = t * QS + wqs * 32 + acc_row(i, g);
            if (q < s.lq) db[(int64_t)q * s.lk] = (TB)ds[i];
          }
        }
      }

      // dV^T += dO^T P and dK^T += Q^T dS (contraction over the 32 queries)
#pragma unroll
      for (int st = 0; st < 16 / KP; ++st) {
        typename E::frag ph, pl, dh, dl;
        if constexpr (KP == 8) {
          ph = pack8(&p[st * 8]);
          dh = pack8(&ds[st * 8]);
          if constexpr (SPLIT) {
            float r1[8], r2[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              r1[j] = p[st * 8 + j] - (float)ph[j];
              r2[j] = ds[st * 8 + j] - (float)dh[j];
            }
            pl = pack8(r1);
            dl = pack8(r2);
          }
        } else {
          ph = p[st];
          dh = ds[st];
        }
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const int off = (d * 32 + l32) * TPITCH + wqs * 32 + g * 16 + st * KP;
          typename E::frag oa, qa;
          if constexpr (KP == 8) {
            oa = *reinterpret_cast<const bf16x8*>(&Ot[off]);
            qa = *reinterpret_cast<const bf16x8*>(&Qt[off]);
          } else {
            oa = Ot[off];
            qa = Qt[off];
          }
          dvacc[d] = E::mma(oa, ph, dvacc[d]);
          dkacc[d] = E::mma(qa, dh, dkacc[d]);
          if constexpr (SPLIT && KP == 8) {
            dvacc[d] = E::mma(oa, pl, dvacc[d]);
            dkacc[d] = E::mma(qa, dl, dkacc[d]);
          }
        }
      }
    }

    TG* kbase = reinterpret_cast<TG*>(a.dk) + koff;
    TG* vbase = reinterpret_cast<TG*>(a.dv) + koff;
    if constexpr (WKQ == 1) {
      if (krow < s.lk) {
        TG* krp = kbase + (int64_t)krow * HD;
        TG* vrp = vbase + (int64_t)krow * HD;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int col = d * 32 + i4 * 8 + g * 4;
            store4<TG>(krp + col, dkacc[d][i4 * 4] * a.scale, dkacc[d][i4 * 4 + 1] * a.scale,
                       dkacc[d][i4 * 4 + 2] * a.scale, dkacc[d][i4 * 4 + 3] * a.scale);
            store4<TG>(vrp + col, dvacc[d][i4 * 4], dvacc[d][i4 * 4 + 1], dvacc[d][i4 * 4 + 2],
                       dvacc[d][i4 * 4 + 3]);
          }
      }
    } else {
      // sum the WKQ query-split partials: part[wave][row][d] with pitch D+1
      float* part = reinterpret_cast<float*>(smem);
      constexpr int P = D + 1;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        __syncthreads();
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            part[(wave * 32 + l32) * P + d * 32 + acc_row(i, g)] = pass == 0 ? dkacc[d][i] : dvacc[d][i];
        __syncthreads();
        const float mul = pass == 0 ? a.scale : 1.0f;
        TG* base = pass == 0 ? kbase : vbase;
        for (int o = tid; o < KT * D; o += kThreads) {
          const int row = o / D, col = o % D;  // row within the unit's key tile
          const int grp = row / 32, r = row % 32;
          float acc = 0.0f;
#pragma unroll
          for (int w2 = 0; w2 < WKQ; ++w2) acc += part[((w2 * WKV + grp) * 32 + r) * P + col];
          const int kr = kt * KT + row;
          if (kr < s.lk) base[(int64_t)kr * HD + col] = (TG)(acc * mul);
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace jattn
