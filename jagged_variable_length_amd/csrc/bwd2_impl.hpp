// dK/dV kernel of jagged attention for bf16 inputs, gfx950, one wave per key
// block (softmax without split operands on 128-key units at D = 128 runs the
// wave-pair kernel instead: bwd_pair_impl.hpp).
//
// Method: "Training GEM at LLM scale" (Meta engineering post), section
// "Jagged Sequence Flash Attention", item "Backward parallelization": dK and
// dV come from their own pass over key tiles (dQ has a separate kernel), so
// every output element has exactly one writer and no atomics are needed.
//
// A unit is (sample, head, key tile of KT = 32*WKV rows).  Each step of the
// unit covers QS = 32*WKQ query rows; wave (wv, wq) takes key block wv and
// query block wq of the step:
//     S  = Q K^T          A = Q rows (LDS), B = K fragments (registers)
//     dP = dO V^T         A = dO rows (LDS), B = V fragments (registers)
//     P  = exp2(S*scale*log2e + bias*log2e - LSE*log2e)   (or act(S*scale+bias))
//     dS = P (dP - Di)                                     (or act'(.) dP)
//     dV^T += dO^T P      A = dO^T via ds_read_b64_tr_b16, B = P in-register
//     dK^T += Q^T dS      A = Q^T  via ds_read_b64_tr_b16, B = dS in-register
//     dBias = dS          (stored straight from registers, one writer)
// A lane owns one key column of S, so P and dS feed the MFMA B operand of the
// dV/dK products without reshuffling (the accumulator rows are queries in the
// order that the transposed reads deliver).
//
// Software pipeline (one wave per SIMD, so nothing else hides latency): the
// S/dP MFMAs of step t+1 are issued interleaved with the VALU work of step t
// (P, dS, dBias), then the dV/dK MFMAs of step t.  A unit starts with the
// S/dP of its step 0 and ends with a step that has no successor.
//
// Memory pipeline: Q, dO, the bias tile and the row statistics of a step go
// HBM -> LDS with buffer loads whose destination is LDS, into a ring of NS
// stages (NS - 2 steps ahead of the step being acquired, also across unit
// boundaries).  K and V of a unit live in registers; the next unit's K/V are
// loaded right after their last S/dP use.  Vector memory operations complete
// in issue order, so each wait lets every operation issued after the needed
// loads stay in flight (exact per-wave counts, dBias stores included).
//
// Sliding window (WIN, section "BlockAttention"): a unit's steps start at the
// first query block whose window reaches its key tile (the plan counts only
// the steps that meet it); P and dS are zeroed element-wise outside the
// window, branch-free inside the interleaved loop.  dBias is not produced
// with a window (its dense [lq, lk] layout would be mostly zeros).
#pragma once
#include <type_traits>

#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"
#include "ring.hpp"

namespace jattn {

template <int D, int WKV, int WKQ, bool SOFTMAX, bool BIAS, bool TWO_ = false>
struct Dkdv2Shape {
  static constexpr int NW = WKV * WKQ;
  static constexpr int KT = 32 * WKV;  // keys per unit
  static constexpr int QS = 32 * WKQ;  // queries per step
  static constexpr int PAD = 2;
  using QT = PadTile<D, PAD>;  // Q and dO rows: pitch = 32 (mod 256) bytes
  static constexpr int Q_BYTES = QT::template bytes<QS>();
  // bias rows (QS queries x KT keys, bf16): pitch = 16 (mod 64) dwords, so
  // the two lane halves (query rows 4 apart) read disjoint banks
  using BT = PadTile<KT, 1>;
  static constexpr int B_BYTES = BIAS ? BT::template bytes<QS>() : 0;
  static constexpr int NRS = SOFTMAX ? 2 * ((QS + 63) / 64) : 0;  // row-stat loads (LSE*log2e, Di)
  static constexpr int RS_BYTES = NRS * 256;
  static constexpr int OFF_O = Q_BYTES;
  static constexpr int OFF_B = 2 * Q_BYTES;
  static constexpr int OFF_RS = OFF_B + B_BYTES;
  static constexpr int STAGE = (OFF_RS + RS_BYTES + 255) / 256 * 256;
  // query-split partials of dK^T (then dV^T) are summed through the stage of
  // the unit's last step, which is free once every wave has computed it
  static constexpr int COMB = WKQ > 1 ? (WKQ - 1) * WKV * D * 32 * 4 : 0;
  // two workgroups per CU (dkdv2_waves_per_simd): each within half the LDS
  static constexpr bool TWO = TWO_;
  static constexpr int NS_FIT = (TWO ? 80 : 160) * 1024 / STAGE;
  static constexpr int NS = NS_FIT >= 4 ? 4 : 3;
  static constexpr int SMEM = NS * STAGE;
  static constexpr int QNI = QT::template ninst<QS>();
  static constexpr int BNI = BIAS ? BT::template ninst<QS>() : 0;
  static_assert(NS_FIT >= 3 && COMB <= STAGE, "LDS budget");
  static_assert(NW == 4, "four waves");
};

// DBIAS: 0 = no dBias, 1 = bf16 dBias, 2 = fp32 dBias
// At D <= 64 without a bias tile or window, on 64- or 128-key units, the
// registers leave room for two waves per SIMD (not with erf-GELU, whose
// derivative needs more): two workgroups per CU, each within half the LDS
// (three stages), and the plan deals the units over twice as many workers
template <int D, bool BIAS, bool WIN, int WKV, int ACT>
constexpr int dkdv2_waves_per_simd() {
  return D <= 64 && !BIAS && !WIN && WKV >= 2 && ACT != kGelu ? 2 : 1;
}

template <typename TG, int D, int WKV, int WKQ, int ACT, bool BIAS, int DBIAS, bool SPLIT, bool WIN = false>
__global__ __launch_bounds__(256, 1) __attribute__((
    amdgpu_waves_per_eu(dkdv2_waves_per_simd<D, BIAS, WIN, WKV, ACT>(), dkdv2_waves_per_simd<D, BIAS, WIN, WKV, ACT>()))) void
dkdv2_kernel(BwdArgs a) {
  static_assert(!WIN || DBIAS == 0, "no dBias with a window");
  // Argument fields as locals: the lambdas below capture by reference, and a
  // reference to the argument block itself would keep it in scratch memory.
  const void* const A_q = a.q;
  const void* const A_k = a.k;
  const void* const A_v = a.v;
  const void* const A_bias = a.bias;
  const void* const A_dout = a.dout;
  const float* const A_di = a.di;
  const float* const A_lse2 = a.lse2;
  void* const A_dk = a.dk;
  void* const A_dv = a.dv;
  void* const A_dbias = a.dbias;
  const int32_t* const A_units = a.units;
  const int32_t* const A_samples = a.samples;
  const int A_H = a.H;
  const float A_scale = a.scale;
  const float A_scale_log2 = a.scale_log2;
  const int64_t A_bias_elems = a.bias_elems;
  const int A_win_l = a.win_l, A_win_r = a.win_r;
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  using Sh = Dkdv2Shape<D, WKV, WKQ, SOFTMAX, BIAS, dkdv2_waves_per_simd<D, BIAS, WIN, WKV, ACT>() == 2>;
  constexpr int NW = Sh::NW, KT = Sh::KT, QS = Sh::QS, ND = D / 32, NKK = D / 16, NS = Sh::NS;
  constexpr int PAD = Sh::PAD;
  constexpr int ESB = DBIAS == 2 ? 4 : 2;  // dBias element size

  __shared__ __attribute__((aligned(1024))) char smem[Sh::SMEM];
  const uint32_t smem_lds = lds_addr(smem);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int wv = wave % WKV, wq = wave / WKV;
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_begin = sload1(a.worker_off, worker);
  const int u_end = sload1(a.worker_off, worker + 1);
  const int H = A_H, HD = A_H * D;

  RowLoader<D, PAD, QS, NW> qload;
  BiasLoader<KT, 1, QS, NW> bload;
  qload.init(wave, lane, HD);
  const uint32_t rs_voff = (uint32_t)lane * H * 4;  // row-stat load: lane l -> query row l of the load

  // Unit record: sample fields only.  Buffer descriptors are rebuilt where
  // they are used (a few scalar operations): three records are live at once
  // (producer, consumer, next), and descriptors in them would spill SGPRs.
  struct Unit {
    int h, kt, n;
    Sample s;
  };
  auto fetch = [&](int u) __attribute__((always_inline)) {
    Unit x;
    const i32x4 un = sload4(A_units, u);
    x.h = un[1];
    x.kt = un[2];
    x.n = un[3];
    x.s = sload_sample(A_samples, un[0]);
    return x;
  };
  // first query row of step t (a windowed unit starts at the first query
  // block whose window reaches its keys)
  auto step_row0 = [&](const Unit& x, int t) __attribute__((always_inline)) {
    return ((WIN ? window_first_step(x.kt * KT, A_win_r, QS) : 0) + t) * QS;
  };
  // window test of slot c (query row rbase + acc_row(c, 0)) against this
  // lane's key, dk = key - rbase: -left <= key - row <= right, row < lq, key < lk
  auto window_ok = [&](const Unit& x, int dk, int rbase, int key, int c) __attribute__((always_inline)) {
    const int off = (c >> 2) * 8 + (c & 3);
    return (uint32_t)(dk - off + A_win_l) <= (uint32_t)(A_win_l + A_win_r) && rbase + off < x.s.lq &&
           key < x.s.lk;
  };

  // ---- producer: the loads of one step into one stage ----
  // The producer cursor (next unit and step to load; units without steps are
  // skipped) runs NS - 2 productions ahead of the step being acquired.  The
  // descriptors of the Q, dO, row-statistic and bias rows are set up once
  // per unit and advanced by a constant per step.
  struct StepDMA {
    uint32_t sb;    // LDS byte address of the stage
    i32x4 rq, rdo;  // Q, dO rows of the step
    i32x4 rs;       // this wave's row-stat load (LSE*log2e or Di)
    i32x4 rb;       // bias rows of the step
    int brows;      // bias rows inside the sample
  };
  constexpr int NJQ = decltype(qload)::NJ, NJB = BIAS ? decltype(bload)::NJ : 0;
  constexpr int NSLOT = 2 * NJQ + (SOFTMAX ? 1 : 0) + NJB;
  static_assert(Sh::NRS <= NW, "one row-stat load per wave at most");
  constexpr int S_OPS = DBIAS != 0 ? 16 : 0;  // dBias stores per step
  // vector memory operations this wave issues per step, and the fewest any wave issues
  const int step_ops = 2 * loads_of(Sh::QNI, wave, NW) + loads_of(Sh::NRS, wave, NW) + loads_of(Sh::BNI, wave, NW);
  constexpr int MIN_OPS =
      2 * loads_of(Sh::QNI, NW - 1, NW) + loads_of(Sh::NRS, NW - 1, NW) + loads_of(Sh::BNI, NW - 1, NW);
  constexpr int LOOK = NS - 2;  // productions in flight at an acquisition
  constexpr int WAIT_N = (LOOK - 1) * MIN_OPS < 63 ? (LOOK - 1) * MIN_OPS : 63;
  // with dBias, the stores of LOOK steps are issued after the oldest
  // production as well in the steady state
  constexpr int WAIT_N2 = WAIT_N + LOOK * S_OPS < 63 ? WAIT_N + LOOK * S_OPS : 63;
  VmLedger<LOOK, WAIT_N, WAIT_N2> ring;

  int pu = u_begin, pt = 0, pn = 0, pst = 0;
  Unit pinfo;
  Walker<false> w_q, w_do, w_rs;  // Q, dO rows and this wave's row-stat rows of the next step
  Walker<true> w_b;               // bias rows of the next step
  int brows = 0;                  // bias rows inside the sample from the next step's first row
  int64_t bstep = 0;              // bytes between consecutive steps' bias rows
  auto start_unit = [&](const Unit& x) __attribute__((always_inline)) {
    const int r0 = step_row0(x, 0);
    const int64_t qo = ((int64_t)(x.s.q0 + r0) * H + x.h) * D * 2;  // first row of step 0
    const int64_t rec = (int64_t)(x.s.lq - r0) * HD * 2;
    w_q.start(A_q, qo, rec);
    w_do.start(A_dout, qo, rec);
    if constexpr (SOFTMAX) {
      // load `wave`: rows 64*(wave % (NRS/2)) .. of LSE (wave < NRS/2) or Di
      constexpr int HALF = Sh::NRS / 2;
      const int jj = wave < Sh::NRS ? wave : 0;
      const int rr = r0 + 64 * (jj % HALF);
      w_rs.start(jj < HALF ? A_lse2 : A_di, ((int64_t)(x.s.q0 + rr) * H + x.h) * 4, (int64_t)(x.s.lq - rr) * H * 4);
    }
    if constexpr (BIAS) {
      // query rows from r0, keys kt*KT .. of the bias block; the offsets follow
      // lk; query rows past the sample end read as zero, like their Q, dO and
      // row statistics: their P is then finite and their dS exactly zero
      bload.init(wave, lane, x.s.lk);
      const int64_t e0 = x.s.bias0 + (int64_t)x.h * x.s.lq * x.s.lk;
      const int64_t off = ((int64_t)r0 * x.s.lk + (int64_t)x.kt * KT) * 2;
      w_b.start(reinterpret_cast<const char*>(A_bias) + e0 * 2, off, (A_bias_elems - e0) * 2 - off);
      brows = x.s.lq - r0;
      bstep = (int64_t)QS * x.s.lk * 2;
    }
  };
  if (pu < u_end) {
    pinfo = fetch(pu);
    pn = pinfo.n;
    if (pn > 0) start_unit(pinfo);
  }
  // slot c (a compile-time constant after unrolling) of this wave's loads
  auto issue_slot = [&](const StepDMA& d, int c) __attribute__((always_inline)) {
    if (c < NJQ) {
      qload.issue_one(c, d.sb, d.rq, wave);
    } else if (c < 2 * NJQ) {
      qload.issue_one(c - NJQ, d.sb + Sh::OFF_O, d.rdo, wave);
    } else if (SOFTMAX && c == 2 * NJQ) {
      if (wave < Sh::NRS) {
        const uint32_t voff = 64 * (wave % (Sh::NRS / 2)) + lane < QS ? rs_voff : 0x80000000u;
        lds_dma4(d.rs, d.sb + Sh::OFF_RS + wave * 256, voff);
      }
    } else if (BIAS && c < NSLOT) {
      bload.issue_one_rows(c - 2 * NJQ - (SOFTMAX ? 1 : 0), d.sb + Sh::OFF_B, d.rb, wave, lane, d.brows);
    }
  };
  auto produce = [&]() __attribute__((always_inline)) {
    if (pt >= pn && pu < u_end) {
      // next unit with steps
      do {
        ++pu;
        if (pu < u_end) pinfo = fetch(pu);
      } while (pu < u_end && pinfo.n == 0);
      pt = 0;
      pn = pu < u_end ? pinfo.n : 0;
      if (pn > 0) start_unit(pinfo);
    }
    if (pt < pn) {
      StepDMA d;
      d.sb = smem_lds + pst * Sh::STAGE;
      d.rq = w_q.words();
      d.rdo = w_do.words();
      if constexpr (SOFTMAX) d.rs = w_rs.words();
      if constexpr (BIAS) {
        d.rb = w_b.words();
        d.brows = brows;
      }
#pragma unroll
      for (int c = 0; c < NSLOT; ++c) issue_slot(d, c);
      w_q.advance(QS * HD * 2);
      w_do.advance(QS * HD * 2);
      if constexpr (SOFTMAX) w_rs.advance(QS * H * 4);
      if constexpr (BIAS) {
        w_b.advance(bstep);
        brows -= QS;
      }
      ++pt;
      pst = pst + 1 == NS ? 0 : pst + 1;
      ring.produced(step_ops);
    } else {
      ring.produced(0);
    }
  };
  // wait until the loads of the step being acquired have landed: everything
  // issued after them may stay in flight (the K/V loads, which the count
  // leaves out, only make the wait stricter)
  auto acquire = [&]() __attribute__((always_inline)) {
    ring.wait_oldest();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // K and V fragments (MFMA B operand) of this lane's key row.  The next unit
  // with steps loads into them right after their last use (the S/dP MFMAs of
  // the unit's last step), before that step's P/dS work and the unit's
  // stores: the wait at their first use then covers neither.  Loads the
  // compiler sees: it waits for them before any use (an asm load's outputs
  // would count as ready at once).
  bf16x8 kf[NKK], vf[NKK];
  auto load_kv = [&](const Unit& x) __attribute__((always_inline)) {
    const int64_t ko = ((int64_t)x.s.k0 * H + x.h) * D;
    const rsrc_t rk = make_rsrc(reinterpret_cast<const bf16*>(A_k) + ko, (uint32_t)x.s.lk * HD * 2);
    const rsrc_t rv = make_rsrc(reinterpret_cast<const bf16*>(A_v) + ko, (uint32_t)x.s.lk * HD * 2);
    const int key = x.kt * KT + wv * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint32_t voff = (uint32_t)(key * HD + kk * 16 + g * 8) * 2;
      kf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rk, voff));
      vf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rv, voff));
    }
  };

  // ---- epilogue: dK = scale * dK^T^T, dV (key-split partials summed) ----
  auto store_unit = [&](const Unit& x, f32x16* dkacc, f32x16* dvacc, int last_stage) __attribute__((always_inline)) {
    float* comb = reinterpret_cast<float*>(smem + last_stage * Sh::STAGE);
    const int key = x.kt * KT + wv * 32 + l32;
    const int64_t ko = ((int64_t)x.s.k0 * H + x.h) * D;
    TG* dkrow = reinterpret_cast<TG*>(A_dk) + ko + (int64_t)key * HD;
    TG* dvrow = reinterpret_cast<TG*>(A_dv) + ko + (int64_t)key * HD;
    const bool valid = key < x.s.lk;
    if (WKQ > 1 && x.n > 0) {
      // partial of query block wq at [slot][d][key]; lane-dependent part in one base
      const int lane_off = g * 4 * 32 + l32;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        f32x16* acc = pass == 0 ? dkacc : dvacc;
        __syncthreads();
        if (wq > 0) {
          float* pw = comb + ((wq - 1) * WKV + wv) * D * 32 + lane_off;
#pragma unroll
          for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i) pw[(d * 32 + (i >> 2) * 8 + (i & 3)) * 32] = acc[d][i];
        }
        __syncthreads();
        if (wq == 0) {
#pragma unroll
          for (int w2 = 1; w2 < WKQ; ++w2) {
            const float* pr = comb + ((w2 - 1) * WKV + wv) * D * 32 + lane_off;
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
              for (int i = 0; i < 16; ++i) acc[d][i] += pr[(d * 32 + (i >> 2) * 8 + (i & 3)) * 32];
          }
        }
      }
    }
    if (wq == 0 && valid) {
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int col = d * 32 + i4 * 8 + g * 4;
          store4<TG>(dkrow + col, dkacc[d][i4 * 4] * A_scale, dkacc[d][i4 * 4 + 1] * A_scale,
                     dkacc[d][i4 * 4 + 2] * A_scale, dkacc[d][i4 * 4 + 3] * A_scale);
          store4<TG>(dvrow + col, dvacc[d][i4 * 4], dvacc[d][i4 * 4 + 1], dvacc[d][i4 * 4 + 2],
                     dvacc[d][i4 * 4 + 3]);
        }
    }
  };

  // ---- phase 1: S = Q K^T and dP = dO V^T of the step in stage st ----
  struct SD {
    f32x16 s, dp;
  };
  auto sdp = [&](int st) __attribute__((always_inline)) {
    const char* qt = smem + st * Sh::STAGE;
    const char* ot = qt + Sh::OFF_O;
    SD r;
    r.s = f32x16{};
    r.dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      r.s = Elem<bf16>::mma(rows_frag<D, PAD>(qt, wq * 32 + l32, kk, g), kf[kk], r.s);
      r.dp = Elem<bf16>::mma(rows_frag<D, PAD>(ot, wq * 32 + l32, kk, g), vf[kk], r.dp);
    }
    return r;
  };

  // ---- phase 2: P, dS (bf16 MFMA operands) and dBias of step t (stage st) ----
  struct Ops {
    bf16x8 ph[2], dh[2], pl[2], dl[2];
  };
  // whether this wave's 32x32 block of step t lies wholly inside the window
  // (its queries and keys inside the sample): then it needs no mask
  auto block_full = [&](const Unit& x, int t) __attribute__((always_inline)) {
    const Window w{A_win_l, A_win_r, x.s.lq, x.s.lk};
    return w.full(step_row0(x, t) + wq * 32, x.kt * KT + wv * 32);
  };
  // bias[q][key] of this lane's key column for its 16 accumulator rows (keys
  // past lk carry the next row's values; only their own, unstored columns see
  // them): the rows of slots 8s .. 8s+7 are the ones a transposed read of
  // step s delivers to the lane (two ds_read_b64_tr_b16 each), in slot order
  auto bias_frag = [&](const char* stage_base, float* out) __attribute__((always_inline)) {
    const char* bt = stage_base + Sh::OFF_B;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 v = trans_frag<KT, 1>(bt, wq, s2, wv * 32, lane);
#pragma unroll
      for (int j = 0; j < 8; ++j) out[s2 * 8 + j] = (float)v[j];
    }
  };
  auto softmax = [&](const Unit& x, int t, int st, const SD& sd) __attribute__((always_inline)) {
    const f32x16 sacc = sd.s, dpacc = sd.dp;
    Ops o;
    const char* qt = smem + st * Sh::STAGE;
    float p[16], ds[16];
    if constexpr (BIAS) bias_frag(qt, p);
    if constexpr (SOFTMAX) {
      const char* rs = qt + Sh::OFF_RS;
      constexpr int DI_OFF = (Sh::NRS / 2) * 256;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int r = wq * 32 + i4 * 8 + g * 4;  // query row within the step
        const int jl = r / 64, rl = r % 64;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(rs + jl * 256 + rl * 4);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(rs + DI_OFF + jl * 256 + rl * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i4 * 4 + j;
          const float c = BIAS ? fmaf(p[i], kLog2e, -l4[j]) : -l4[j];
          p[i] = fast_exp2(fmaf(sacc[i], A_scale_log2, c));
          ds[i] = p[i] * (dpacc[i] - d4[j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float xv = BIAS ? fmaf(sacc[i], A_scale, p[i]) : sacc[i] * A_scale;
        p[i] = act_fwd(ACT, xv);
        ds[i] = act_grad(ACT, xv) * dpacc[i];
      }
    }
    if (WIN && !block_full(x, t)) {
      const int key = x.kt * KT + wv * 32 + l32;
      const int rbase = step_row0(x, t) + wq * 32 + g * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = window_ok(x, key - rbase, rbase, key, i);
        p[i] = ok ? p[i] : 0.0f;
        ds[i] = ok ? ds[i] : 0.0f;
      }
    }
    if constexpr (DBIAS != 0) {
      // dBias[q][key] = dS; rows past the sample end fall outside the
      // descriptor, and a lane whose key is past the end stores out of range
      const int key = x.kt * KT + wv * 32 + l32;
      const rsrc_t rdbr = make_rsrc(reinterpret_cast<const char*>(A_dbias) +
                                        (x.s.bias0 + (int64_t)x.h * x.s.lq * x.s.lk) * ESB,
                                    (uint32_t)x.s.lq * x.s.lk * ESB);
      const uint32_t vb = key < x.s.lk ? (uint32_t)(((step_row0(x, t) + wq * 32 + g * 4) * x.s.lk + key) * ESB)
                                       : 0x80000000u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t voff = vb + (uint32_t)(((i >> 2) * 8 + (i & 3)) * x.s.lk * ESB);
        if constexpr (DBIAS == 2)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ds[i]), rdbr, voff, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16)ds[i]), rdbr, voff, 0, 0);
      }
      ring.counted(S_OPS);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      o.ph[s2] = pack8(&p[s2 * 8]);
      o.dh[s2] = pack8(&ds[s2 * 8]);
      if constexpr (SPLIT) {
        float r1[8], r2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          r1[j] = p[s2 * 8 + j] - (float)o.ph[s2][j];
          r2[j] = ds[s2 * 8 + j] - (float)o.dh[s2][j];
        }
        o.pl[s2] = pack8(r1);
        o.dl[s2] = pack8(r2);
      }
    }
    return o;
  };

  // ---- phase 3: dV^T += dO^T P, dK^T += Q^T dS from stage st ----
  auto dkdv_mma = [&](int st, const Ops& o, f32x16* dkacc, f32x16* dvacc) __attribute__((always_inline)) {
    const char* qt = smem + st * Sh::STAGE;
    const char* ot = qt + Sh::OFF_O;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const bf16x8 oa = trans_frag<D, PAD>(ot, wq, s2, d * 32, lane);
        const bf16x8 qa = trans_frag<D, PAD>(qt, wq, s2, d * 32, lane);
        dvacc[d] = Elem<bf16>::mma(oa, o.ph[s2], dvacc[d]);
        dkacc[d] = Elem<bf16>::mma(qa, o.dh[s2], dkacc[d]);
        if constexpr (SPLIT) {
          dvacc[d] = Elem<bf16>::mma(oa, o.pl[s2], dvacc[d]);
          dkacc[d] = Elem<bf16>::mma(qa, o.dl[s2], dkacc[d]);
        }
      }
    }
  };

  // ---- phases 1 + 2 fused: S/dP of the step in stage cn, written out so
  // that each of its 16 MFMAs is followed by the VALU work of one element of
  // P/dS (and its dBias store) of step t in stage cs; a scheduling fence
  // after each pair keeps that order, so the matrix core and the VALU work
  // side by side.  Operand LDS reads run two MFMAs ahead.
  // MASK (windowed kernels): apply the window mask to P and dS; instances
  // with and without it keep the interleaved loop free of branches
  auto sdp_softmax = [&](auto mask_tag, int cn, const Unit& x, int t, int cs_, const SD& cur, SD& nx,
                         Ops& o) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* qn = smem + cn * Sh::STAGE;
    const char* on = qn + Sh::OFF_O;
    const char* qt = smem + cs_ * Sh::STAGE;
    float bias[16], lse[16], di[16];
    if constexpr (BIAS) bias_frag(qt, bias);
    if constexpr (SOFTMAX) {
      const char* rs = qt + Sh::OFF_RS;
      constexpr int DI_OFF = (Sh::NRS / 2) * 256;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int r = wq * 32 + i4 * 8 + g * 4;
        const int jl = r / 64, rl = r % 64;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(rs + jl * 256 + rl * 4);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(rs + DI_OFF + jl * 256 + rl * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lse[i4 * 4 + j] = l4[j];
          di[i4 * 4 + j] = d4[j];
        }
      }
    }
    // dBias[q][key] = dS; rows past the sample end fall outside the
    // descriptor, and a lane whose key is past the end stores out of range
    uint32_t vb = 0;
    if constexpr (DBIAS != 0) {
      const int key = x.kt * KT + wv * 32 + l32;
      vb = key < x.s.lk ? (uint32_t)(((step_row0(x, t) + wq * 32 + g * 4) * x.s.lk + key) * ESB) : 0x80000000u;
    }
    const int wkey = x.kt * KT + wv * 32 + l32;
    const int wrbase = WIN ? step_row0(x, t) + wq * 32 + g * 4 : 0;
    bf16x8 qa[NKK], oa[NKK];
    qa[0] = rows_frag<D, PAD>(qn, wq * 32 + l32, 0, g);
    oa[0] = rows_frag<D, PAD>(on, wq * 32 + l32, 0, g);
    if constexpr (NKK > 1) {
      qa[1] = rows_frag<D, PAD>(qn, wq * 32 + l32, 1, g);
      oa[1] = rows_frag<D, PAD>(on, wq * 32 + l32, 1, g);
    }
    nx.s = f32x16{};
    nx.dp = f32x16{};
    float p[16], ds[16];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int kk = c / 2 % NKK;
      if (c < 2 * NKK) {
        if (c % 2 == 0) {
          nx.s = Elem<bf16>::mma(qa[kk], kf[kk], nx.s);
          if (kk + 2 < NKK) qa[kk + 2] = rows_frag<D, PAD>(qn, wq * 32 + l32, kk + 2, g);
        } else {
          nx.dp = Elem<bf16>::mma(oa[kk], vf[kk], nx.dp);
          if (kk + 2 < NKK) oa[kk + 2] = rows_frag<D, PAD>(on, wq * 32 + l32, kk + 2, g);
        }
      }

      // element c of P and dS of step t
      const float sv = cur.s[c], dpv = cur.dp[c];
      if constexpr (SOFTMAX) {
        const float cc = BIAS ? fmaf(bias[c], kLog2e, -lse[c]) : -lse[c];
        p[c] = fast_exp2(fmaf(sv, A_scale_log2, cc));
        ds[c] = p[c] * (dpv - di[c]);
      } else {
        const float xv = BIAS ? fmaf(sv, A_scale, bias[c]) : sv * A_scale;
        p[c] = act_fwd(ACT, xv);
        ds[c] = act_grad(ACT, xv) * dpv;
      }
      if constexpr (MASK) {
        const bool ok = window_ok(x, wkey - wrbase, wrbase, wkey, c);
        p[c] = ok ? p[c] : 0.0f;
        ds[c] = ok ? ds[c] : 0.0f;
      }
      if constexpr (DBIAS != 0) {
        const rsrc_t rdbr = make_rsrc(
            reinterpret_cast<const char*>(A_dbias) + (x.s.bias0 + (int64_t)x.h * x.s.lq * x.s.lk) * ESB,
            (uint32_t)x.s.lq * x.s.lk * ESB);
        const uint32_t voff = vb + (uint32_t)(((c >> 2) * 8 + (c & 3)) * x.s.lk * ESB);
        if constexpr (DBIAS == 2)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ds[c]), rdbr, voff, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16)ds[c]), rdbr, voff, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DBIAS != 0) ring.counted(S_OPS);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      o.ph[s2] = pack8(&p[s2 * 8]);
      o.dh[s2] = pack8(&ds[s2 * 8]);
      if constexpr (SPLIT) {
        float r1[8], r2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          r1[j] = p[s2 * 8 + j] - (float)o.ph[s2][j];
          r2[j] = ds[s2 * 8 + j] - (float)o.dh[s2][j];
        }
        o.pl[s2] = pack8(r1);
        o.dl[s2] = pack8(r2);
      }
    }
  };

  // The bias tensor's last element may straddle the end of its range by half
  // a dword, which the range check drops.  In the step that holds it (the
  // last step of the last key tile of the tensor's last (sample, head)),
  // one lane writes it into the bias tile after the tile has landed; a
  // second barrier publishes it.  Called after every acquisition, outside
  // the branch-free compute region.
  auto patch_tail = [&](const Unit& x, int t, int st) __attribute__((always_inline)) {
    if constexpr (BIAS) {
      if (t + 1 == x.n && x.s.bias0 + (int64_t)(x.h + 1) * x.s.lq * x.s.lk == A_bias_elems &&
          (x.s.lk - 1) / KT == x.kt) {
        if (wave == 0 && lane == 0) {
          const rsrc_t rl = make_rsrc(reinterpret_cast<const bf16*>(A_bias) + (A_bias_elems - 1), 2);
          const uint16_t last = buf_load2(rl, 0);
          char* bt = smem + st * Sh::STAGE + Sh::OFF_B;
          *reinterpret_cast<uint16_t*>(bt + ((x.s.lq - 1) - step_row0(x, t)) * Sh::BT::PITCH +
                                       ((x.s.lk - 1) - x.kt * KT) * 2) = last;
        }
        __syncthreads();
      }
    }
  };

  // ---- consumer ----
  if (u_begin >= u_end) return;
  for (int j = 0; j < LOOK; ++j) produce();
  // first unit with steps: its K/V
  for (int u0 = u_begin; u0 < u_end; ++u0) {
    const Unit x0 = fetch(u0);
    if (x0.n > 0) {
      load_kv(x0);
      break;
    }
  }

  int cs = 0;  // stage of the step whose P/dS is computed next
  for (int u = u_begin; u < u_end; ++u) {
    const Unit x = fetch(u);
    f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      dkacc[d] = f32x16{};
      dvacc[d] = f32x16{};
    }
    if (x.n > 0) {
      // prologue: S/dP of step 0
      acquire();
      produce();
      patch_tail(x, 0, cs);
      SD cur = sdp(cs);
      for (int t = 0; t + 1 < x.n; ++t) {
        // S/dP of step t+1 (stage cn) beside P/dS of step t (stage cs)
        const int cn = cs + 1 == NS ? 0 : cs + 1;
        acquire();
        produce();
        patch_tail(x, t + 1, cn);
        SD nxt;
        Ops ops;
        if (WIN && !block_full(x, t))
          sdp_softmax(std::true_type{}, cn, x, t, cs, cur, nxt, ops);
        else
          sdp_softmax(std::false_type{}, cn, x, t, cs, cur, nxt, ops);
        dkdv_mma(cs, ops, dkacc, dvacc);
        cur = nxt;
        cs = cn;
      }
      // K/V are free: the next unit with steps loads its own
      for (int un = u + 1; un < u_end; ++un) {
        const Unit xn = fetch(un);
        if (xn.n > 0) {
          load_kv(xn);
          break;
        }
      }
      dkdv_mma(cs, softmax(x, x.n - 1, cs, cur), dkacc, dvacc);
    }
    store_unit(x, dkacc, dvacc, cs);
    if (x.n > 0) cs = cs + 1 == NS ? 0 : cs + 1;
  }
  // every production was acquired; only stores and register loads can still
  // be in flight
  wait_vmcnt<0>();
}

}  // namespace jattn
