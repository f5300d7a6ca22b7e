// dK/dV kernel with a wave pair per key block: bf16 inputs, softmax over a
// dense mask or a sliding window, 128-key units, gfx950.
//
// Method: "Training GEM at LLM scale" (Meta engineering post), section
// "Jagged Sequence Flash Attention", item "Backward parallelization": dK and
// dV come from their own pass over key tiles, one writer per output element
// and no atomics; items "Warp specialization and persistent kernels": waves
// of a workgroup take different roles.
//
// A unit is (sample, head, key tile of 128 rows); each step covers 32 query
// rows.  Each of the four 32-key blocks of the tile has two waves, so a
// workgroup has eight (two per SIMD, which is what the pairing buys: the
// registers one wave needs for a key block, the dK^T and dV^T accumulators
// and both K and V fragments, leave room for one wave per SIMD only):
//   P wave  (waves 0-3): S = Q K^T (K fragments in registers),
//                        P = exp2(S*scale*log2e + bias*log2e - LSE*log2e),
//                        dV^T += dO^T P; P (fp32) goes to the partner
//                        through LDS.
//   dS wave (waves 4-7): dP = dO V^T (V fragments in registers); one step
//                        later, with that step's P from the partner:
//                        dS = P (dP - Di), dBias = dS, dK^T += Q^T dS.
// Both waves use the same 32x32 accumulator layout (lane = key column, 16
// query rows), so the hand-over is a lane-private 64-byte record per lane
// (fp32, so that dS is formed from P before its rounding to the bf16 MFMA
// operand, as in the single-wave kernel).
// The dS wave's MFMAs for dP of step t are written interleaved with its VALU
// work on dS of step t - 1 (with dBias its stores hold that order; without
// them the compiler may issue the MFMAs first).
//
// Sliding window (WIN, section "BlockAttention"): a unit's steps start at the
// first query block whose window reaches its keys; the P wave zeroes P
// outside the window, which makes dS zero there as well (no dBias).
//
// Memory pipeline: the ring of the single-wave kernel (Q, dO, bias tile and
// row statistics of a step loaded HBM -> LDS ahead of use, NS - 2 steps in
// flight, exact per-wave vmcnt waits), with its loads dealt over the eight
// waves.  A stage is read in the iteration that acquires it and, by the dS
// wave, in the next one.  P records are double-buffered: the one written in
// step t is read after the barrier of step t + 1 and rewritten after the
// barrier of step t + 2.  A unit ends with one more barrier, after which the
// dS waves finish its last step.
#pragma once

#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"
#include "ring.hpp"

namespace jattn {

template <int D, bool BIAS>
struct DkdvPairShape {
  static constexpr int NW = 8;   // waves
  static constexpr int KB = 4;   // 32-key blocks per unit
  static constexpr int KT = 32 * KB;
  static constexpr int QS = 32;  // queries per step
  // Q and dO rows with three spare 16-byte slots: the row pitch moves the
  // 16-byte chunk of consecutive rows by 12 banks, so the 16 rows of a
  // ds_read_b128 group fall on distinct banks, and the 4 rows of a
  // transposed-read group on disjoint 8-bank spans
  static constexpr int PAD = D == 128 ? 3 : 2;
  using QT = PadTile<D, PAD>;
  static constexpr int Q_BYTES = QT::template bytes<QS>();
  using BT = PadTile<KT, 1>;
  static constexpr int B_BYTES = BIAS ? BT::template bytes<QS>() : 0;
  static constexpr int NRS = 2;  // row-stat loads: LSE*log2e, Di (32 rows each)
  static constexpr int OFF_O = Q_BYTES;
  static constexpr int OFF_B = 2 * Q_BYTES;
  static constexpr int OFF_RS = OFF_B + B_BYTES;
  static constexpr int STAGE = (OFF_RS + NRS * 256 + 255) / 256 * 256;
  static constexpr int PREC = 64 * 64;              // one key block's P record: 64 bytes per lane
  static constexpr int PX_BYTES = 2 * KB * PREC;    // two buffers
  static constexpr int NS_FIT = (160 * 1024 - PX_BYTES) / STAGE;
  static constexpr int NS = NS_FIT >= 4 ? 4 : 3;
  static constexpr int OFF_PX = NS * STAGE;
  static constexpr int SMEM = OFF_PX + PX_BYTES;
  static constexpr int QNI = QT::template ninst<QS>();
  static constexpr int BNI = BIAS ? BT::template ninst<QS>() : 0;
  static_assert(NS_FIT >= 3, "LDS budget");
};

// DBIAS: 0 = no dBias, 1 = bf16 dBias, 2 = fp32 dBias
template <typename TG, int D, bool BIAS, int DBIAS, bool WIN = false>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkdv_pair_kernel(BwdArgs a) {
  static_assert(BIAS || DBIAS == 0, "dBias needs a bias");
  static_assert(!WIN || DBIAS == 0, "no dBias with a window");
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
  using Sh = DkdvPairShape<D, BIAS>;
  constexpr int NW = Sh::NW, KT = Sh::KT, QS = Sh::QS, ND = D / 32, NKK = D / 16, NS = Sh::NS;
  constexpr int PAD = Sh::PAD;
  constexpr int ESB = DBIAS == 2 ? 4 : 2;  // dBias element size

  __shared__ __attribute__((aligned(1024))) char smem[Sh::SMEM];
  const uint32_t smem_lds = lds_addr(smem);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int role = wave / Sh::KB;  // 0: P wave, 1: dS wave
  const int wv = wave % Sh::KB;    // key block
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_begin = sload1(a.worker_off, worker);
  const int u_end = sload1(a.worker_off, worker + 1);
  const int H = A_H, HD = A_H * D;

  RowLoader<D, PAD, QS, NW> qload;
  BiasLoader<KT, 1, QS, NW> bload;
  qload.init(wave, lane, HD);
  const uint32_t rs_voff = (uint32_t)lane * H * 4;  // row-stat load: lane l -> query row l

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

  // ---- producer (as in the single-wave kernel, loads over eight waves) ----
  struct StepDMA {
    uint32_t sb;
    i32x4 rq, rdo, rs, rb;
    int brows;
  };
  constexpr int NJQ = decltype(qload)::NJ, NJB = BIAS ? decltype(bload)::NJ : 0;
  constexpr int NSLOT = 2 * NJQ + 1 + NJB;
  constexpr int S_OPS = DBIAS != 0 ? 16 : 0;  // dBias stores of a dS wave per step
  const int step_ops = 2 * loads_of(Sh::QNI, wave, NW) + loads_of(Sh::NRS, wave, NW) + loads_of(Sh::BNI, wave, NW);
  constexpr int MIN_OPS =
      2 * loads_of(Sh::QNI, NW - 1, NW) + loads_of(Sh::NRS, NW - 1, NW) + loads_of(Sh::BNI, NW - 1, NW);
  constexpr int LOOK = NS - 2;
  constexpr int WAIT_N = (LOOK - 1) * MIN_OPS < 63 ? (LOOK - 1) * MIN_OPS : 63;
  // a dS wave with dBias has, in the steady state, the stores of LOOK steps
  // issued after the oldest production as well
  constexpr int WAIT_N2 = WAIT_N + LOOK * S_OPS < 63 ? WAIT_N + LOOK * S_OPS : 63;
  VmLedger<LOOK, WAIT_N, WAIT_N2> ring;

  int pu = u_begin, pt = 0, pn = 0, pst = 0;
  Unit pinfo;
  Walker<false> w_q, w_do, w_rs;
  Walker<true> w_b;
  int brows = 0;
  int64_t bstep = 0;
  // first query row of step t (a windowed unit starts at the first query
  // block whose window reaches its keys; the plan counts only those steps)
  auto step_row0 = [&](const Unit& x, int t) __attribute__((always_inline)) {
    return ((WIN ? window_first_step(x.kt * KT, A_win_r, QS) : 0) + t) * QS;
  };
  auto start_unit = [&](const Unit& x) __attribute__((always_inline)) {
    const int r0 = step_row0(x, 0);
    const int64_t qo = ((int64_t)(x.s.q0 + r0) * H + x.h) * D * 2;
    const int64_t rec = (int64_t)(x.s.lq - r0) * HD * 2;
    w_q.start(A_q, qo, rec);
    w_do.start(A_dout, qo, rec);
    // wave 0 loads LSE*log2e rows, wave 1 Di rows
    w_rs.start(wave == 0 ? A_lse2 : A_di, ((int64_t)(x.s.q0 + r0) * H + x.h) * 4, (int64_t)(x.s.lq - r0) * H * 4);
    if constexpr (BIAS) {
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
  auto issue_slot = [&](const StepDMA& d, int c) __attribute__((always_inline)) {
    if (c < NJQ) {
      qload.issue_one(c, d.sb, d.rq, wave);
    } else if (c < 2 * NJQ) {
      qload.issue_one(c - NJQ, d.sb + Sh::OFF_O, d.rdo, wave);
    } else if (c == 2 * NJQ) {
      if (wave < Sh::NRS) lds_dma4(d.rs, d.sb + Sh::OFF_RS + wave * 256, lane < QS ? rs_voff : 0x80000000u);
    } else if (BIAS && c < NSLOT) {
      bload.issue_one_rows(c - 2 * NJQ - 1, d.sb + Sh::OFF_B, d.rb, wave, lane, d.brows);
    }
  };
  auto produce = [&]() __attribute__((always_inline)) {
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
      StepDMA d;
      d.sb = smem_lds + pst * Sh::STAGE;
      d.rq = w_q.words();
      d.rdo = w_do.words();
      d.rs = w_rs.words();
      if constexpr (BIAS) {
        d.rb = w_b.words();
        d.brows = brows;
      }
#pragma unroll
      for (int c = 0; c < NSLOT; ++c) issue_slot(d, c);
      w_q.advance(QS * HD * 2);
      w_do.advance(QS * HD * 2);
      w_rs.advance(QS * H * 4);
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
  auto acquire = [&]() __attribute__((always_inline)) {
    ring.wait_oldest();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // the bias tensor's last element (see the single-wave kernel): patched into
  // the tile of the step that holds it, after the tile has landed
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
  auto next_stage = [](int s) __attribute__((always_inline)) { return s + 1 == NS ? 0 : s + 1; };

  // K (P waves) or V (dS waves) fragments, MFMA B operand, of this lane's key
  // row.  Loads the compiler sees: it waits for them before the first use,
  // which is outside every step loop (the first step of a unit is peeled).
  bf16x8 kvf[NKK];
  auto load_kv = [&](const Unit& x) __attribute__((always_inline)) {
    const int64_t ko = ((int64_t)x.s.k0 * H + x.h) * D;
    const bf16* src = reinterpret_cast<const bf16*>(role == 0 ? A_k : A_v) + ko;
    const rsrc_t r = make_rsrc(src, (uint32_t)x.s.lk * HD * 2);
    const int key = x.kt * KT + wv * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      kvf[kk] = __builtin_bit_cast(bf16x8, buf_load16(r, (uint32_t)(key * HD + kk * 16 + g * 8) * 2));
  };
  // the next unit with steps (after u) loads its fragments
  auto load_next_kv = [&](int u) __attribute__((always_inline)) {
    for (int un = u + 1; un < u_end; ++un) {
      const Unit xn = fetch(un);
      if (xn.n > 0) {
        load_kv(xn);
        break;
      }
    }
  };

  // dP = dO V^T of the step in stage st (dS wave)
  auto rows_mma = [&](int st) __attribute__((always_inline)) {
    const char* t = smem + st * Sh::STAGE + Sh::OFF_O;
    // every operand read issued before the first MFMA of the chain
    bf16x8 fr[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) fr[kk] = rows_frag<D, PAD>(t, l32, kk, g);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) acc = Elem<bf16>::mma(fr[kk], kvf[kk], acc);
    return acc;
  };
  // acc[d] += X^T Y for the 32 rows of stage st's tile X (Q or dO), Y = the
  // packed bf16 operand (P or dS) of this lane's key column
  // (every operand read issued before the first MFMA: left to the compiler
  // at this register pressure, each MFMA waits for its own read)
  auto trans_mma = [&](const char* x, const bf16x8* y, f32x16* acc) __attribute__((always_inline)) {
    bf16x8 xa[2][ND];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d = 0; d < ND; ++d) xa[s2][d] = trans_frag<D, PAD>(x, 0, s2, d * 32, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[d] = Elem<bf16>::mma(xa[s2][d], y[s2], acc[d]);
  };
  char* const px = smem + Sh::OFF_PX + wv * Sh::PREC + lane * 16;

  // ---- P wave, step t (stage st): S = Q K^T, P, hand-over, dV^T += dO^T P.
  // The LDS reads that S and P need are all issued while the S MFMAs run
  // (left to the compiler, the row statistics and bias are read after them,
  // each waited for on its own); with LOAD the next unit's K fragments load
  // right after the S MFMAs, their last use ----
  auto p_step = [&](auto load_tag, const Unit& x, int u, int t, int st, f32x16* acc) __attribute__((always_inline)) {
    constexpr bool LOAD = decltype(load_tag)::value;
    const char* qt = smem + st * Sh::STAGE;
    bf16x8 fr[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) fr[kk] = rows_frag<D, PAD>(qt, l32, kk, g);
    __builtin_amdgcn_sched_barrier(0);
    // the row statistics and bias values are read once half of the S
    // operands have been consumed (registers), ahead of the other half
    constexpr int KH = NKK / 2;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) sacc = Elem<bf16>::mma(fr[kk], kvf[kk], sacc);
    f32x4 l4[4];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) l4[i4] = *reinterpret_cast<const f32x4*>(qt + Sh::OFF_RS + (i4 * 8 + g * 4) * 4);
    // bias[q][key] of this lane's key column in accumulator row order
    bf16x8 bv[2];
    if constexpr (BIAS) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) bv[s2] = trans_frag<KT, 1>(qt + Sh::OFF_B, 0, s2, wv * 32, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = KH; kk < NKK; ++kk) sacc = Elem<bf16>::mma(fr[kk], kvf[kk], sacc);
    if constexpr (LOAD) load_next_kv(u);
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float lse = l4[i / 4][i % 4];
      const float c = BIAS ? fmaf((float)bv[i / 8][i % 8], kLog2e, -lse) : -lse;
      p[i] = fast_exp2(fmaf(sacc[i], A_scale_log2, c));
    }
    if constexpr (WIN) {
      // P of pairs outside the window (and of rows or keys past the sample)
      // is zero; the dS wave's dS = P (dP - Di) then is too.  A uniform
      // branch skips the test for blocks wholly inside the window.
      const int rbase = step_row0(x, t) + g * 4;
      const int key = x.kt * KT + wv * 32 + l32;
      const Window w{A_win_l, A_win_r, x.s.lq, x.s.lk};
      if (!w.full(step_row0(x, t), x.kt * KT + wv * 32)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = w.allows(rbase + (i >> 2) * 8 + (i & 3), key) ? p[i] : 0.0f;
      }
    }
    char* rec = px + (t & 1) * Sh::KB * Sh::PREC;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4*>(rec + j * 1024) = f32x4{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
    bf16x8 ph[2];
    ph[0] = pack8(&p[0]);
    ph[1] = pack8(&p[8]);
    trans_mma(qt + Sh::OFF_O, ph, acc);
  };

  // ---- dS wave: dS of step tp (stage sp) from its dP and the partner's P;
  // with NEXT, dP of the step in stage sn is issued alongside (its MFMAs
  // interleaved with the element-wise work, two elements per MFMA) ----
  auto ds_step = [&](auto next_tag, const Unit& x, int tp, int sp, const f32x16& dp, int sn, f32x16& dpn,
                     f32x16* acc) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    const char* qt = smem + sp * Sh::STAGE;
    const char* on = smem + sn * Sh::STAGE + Sh::OFF_O;
    const char* rec = px + (tp & 1) * Sh::KB * Sh::PREC;
    f32x4 pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = *reinterpret_cast<const f32x4*>(rec + j * 1024);
    float di[16];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(qt + Sh::OFF_RS + 256 + (i4 * 8 + g * 4) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) di[i4 * 4 + j] = d4[j];
    }
    // dBias[q][key] = dS; rows past the sample end fall outside the
    // descriptor, and a lane whose key is past the end stores out of range
    uint32_t vb = 0;
    if constexpr (DBIAS != 0) {
      const int key = x.kt * KT + wv * 32 + l32;
      vb = key < x.s.lk ? (uint32_t)(((tp * QS + g * 4) * x.s.lk + key) * ESB) : 0x80000000u;
    }
    bf16x8 oa[NKK];
    if constexpr (NEXT) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) oa[kk] = rows_frag<D, PAD>(on, l32, kk, g);
      dpn = f32x16{};
    }
    float ds[16];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if constexpr (NEXT) {
        if (c % 2 == 0 && c / 2 < NKK) {
          const int kk = c / 2;
          dpn = Elem<bf16>::mma(oa[kk], kvf[kk], dpn);
        }
      }
      ds[c] = pr[c / 4][c % 4] * (dp[c] - di[c]);
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
    bf16x8 dh[2];
    dh[0] = pack8(&ds[0]);
    dh[1] = pack8(&ds[8]);
    trans_mma(qt, dh, acc);
  };

  // ---- epilogue: dV (P waves) or dK = scale * dK^T^T (dS waves) ----
  auto store_unit = [&](const Unit& x, const f32x16* acc) __attribute__((always_inline)) {
    const int key = x.kt * KT + wv * 32 + l32;
    if (key >= x.s.lk) return;
    const int64_t ko = ((int64_t)x.s.k0 * H + x.h) * D;
    TG* row = reinterpret_cast<TG*>(role == 0 ? A_dv : A_dk) + ko + (int64_t)key * HD;
    const float sc = role == 0 ? 1.0f : A_scale;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        store4<TG>(row + d * 32 + i4 * 8 + g * 4, acc[d][i4 * 4] * sc, acc[d][i4 * 4 + 1] * sc,
                   acc[d][i4 * 4 + 2] * sc, acc[d][i4 * 4 + 3] * sc);
  };

  // ---- consumer ----
  if (u_begin >= u_end) return;
  for (int j = 0; j < LOOK; ++j) produce();
  for (int u0 = u_begin; u0 < u_end; ++u0) {
    const Unit x0 = fetch(u0);
    if (x0.n > 0) {
      load_kv(x0);
      break;
    }
  }

  int cs = 0;  // stage of the next step to acquire
  for (int u = u_begin; u < u_end; ++u) {
    const Unit x = fetch(u);
    f32x16 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = f32x16{};
    if (x.n > 0) {
      acquire();
      produce();
      patch_tail(x, 0, cs);
      if (role == 0) {
        if (x.n == 1) {
          p_step(std::true_type{}, x, u, 0, cs, acc);
          cs = next_stage(cs);
        } else {
          p_step(std::false_type{}, x, u, 0, cs, acc);
          cs = next_stage(cs);
          for (int t = 1; t + 1 < x.n; ++t) {
            acquire();
            produce();
            patch_tail(x, t, cs);
            p_step(std::false_type{}, x, u, t, cs, acc);
            cs = next_stage(cs);
          }
          acquire();
          produce();
          patch_tail(x, x.n - 1, cs);
          p_step(std::true_type{}, x, u, x.n - 1, cs, acc);
          cs = next_stage(cs);
        }
        // the partner reads P of the unit's last step after this barrier
        __syncthreads();
      } else {
        f32x16 dp = rows_mma(cs), dpn;
        if (x.n == 1) {
          load_next_kv(u);
          __syncthreads();
          ds_step(std::false_type{}, x, 0, cs, dp, cs, dpn, acc);
          cs = next_stage(cs);
        } else {
          int sp = cs;
          cs = next_stage(cs);
          for (int t = 1; t + 1 < x.n; ++t) {
            acquire();
            produce();
            patch_tail(x, t, cs);
            ds_step(std::true_type{}, x, t - 1, sp, dp, cs, dpn, acc);
            dp = dpn;
            sp = cs;
            cs = next_stage(cs);
          }
          acquire();
          produce();
          patch_tail(x, x.n - 1, cs);
          ds_step(std::true_type{}, x, x.n - 2, sp, dp, cs, dpn, acc);
          load_next_kv(u);
          __syncthreads();
          ds_step(std::false_type{}, x, x.n - 1, cs, dpn, cs, dp, acc);
          cs = next_stage(cs);
        }
      }
    }
    store_unit(x, acc);
  }
  // every production was acquired; only stores and register loads can still
  // be in flight
  wait_vmcnt<0>();
}

}  // namespace jattn
