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
// destination is LDS (no registers, rows past the sample end read as zero)
// into a ring of NS stages: a producer cursor runs ahead of the step being
// computed, across unit boundaries, and each step waits only for its own
// loads (per-wave counts); one barrier per step.  With three stages or more
// the steps are software-pipelined: the S^T MFMAs of step t+1 are issued
// between the exponentials of step t's softmax, then P V of step t.  K and V rows are stored
// permuted within each 32-key block (RowLoader PERM), which makes the 16
// scores a lane holds 16 consecutive keys: the lane's bias values are then
// two aligned 16-byte LDS reads.  The key-split partials of one query group
// are combined through LDS at the end of a unit.
//
// Sliding window (WIN, section "BlockAttention"): the unit's steps start at
// the first key tile its window meets (the plan counts only the steps that
// meet it); 32x32 blocks that are not wholly inside the window, or that hold
// keys past the sample end, are masked element-wise, so no padding
// correction is needed.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"
#include "ring.hpp"

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
  using BT = PadTile<BN, 1>;  // bias rows: pitch = 16 (mod 256) bytes, 16-byte reads conflict-free
  static constexpr int B_BYTES = BIAS ? BT::template bytes<BM>() : 0;
  static constexpr int STAGE = K_BYTES + V_BYTES + B_BYTES;
  // ring depth: up to four stages (three steps in flight beside the one computed)
  static constexpr int NS_FIT = 160 * 1024 / STAGE;
  static constexpr int NS = NS_FIT >= 4 ? 4 : NS_FIT;
  static_assert(NS >= 2, "two stages at least");
  // LDS-destination load instructions of one step (whole workgroup)
  static constexpr int KNI = KT::template ninst<BN>();
  static constexpr int VNI = VT::template ninst<BN>();
  static constexpr int BNI = BIAS ? BT::template ninst<BM>() : 0;
  // The key-split partials of O (key blocks 1..WK-1) are summed through the
  // stage of the unit's last step, DP 32-column blocks of D per pass; their
  // m, l, l_rounded go first.
  static constexpr int STATS = (WK - 1) * WQ * 32 * 3 * 4;
  static constexpr int COMB_PER_D = (WK - 1) * WQ * 32 * 32 * 4;
  static constexpr int DP_FIT = WK > 1 ? (STAGE - STATS) / COMB_PER_D : ND;
  // One pass through a region of its own when the LDS budget allows (no
  // extra barriers: short-key units are often a single step), else passes
  // through the free stage.
  static constexpr int OWN = STATS + COMB_PER_D * ND;
  static constexpr bool COMB_IN_STAGE = WK > 1 && NS * STAGE + OWN > 160 * 1024;
  static_assert(!COMB_IN_STAGE || DP_FIT >= 1, "combine pass does not fit a stage");
  static constexpr int DP = !COMB_IN_STAGE || DP_FIT >= ND ? ND : (DP_FIT >= 2 && ND % 2 == 0 ? 2 : 1);
  static constexpr int EXTRA = (WK > 1 && !COMB_IN_STAGE) ? OWN : 0;
  static constexpr int SMEM = NS * STAGE + EXTRA;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
};

// 4 query groups x one key block without a bias or window run three
// workgroups per CU at D <= 64 and two at D = 128 (the plan gives that shape
// three or two times the workers); the other shapes keep the default (at
// least one)
template <int D, int WQ, int WK, bool BIAS, bool WIN>
constexpr int fwd2_waves_per_simd() {
  return WQ == 4 && WK == 1 && !BIAS && !WIN ? (D <= 64 ? 3 : 2) : 1;
}

template <typename TO, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT, bool WIN = false>
__global__ __launch_bounds__(64 * WQ * WK, (fwd2_waves_per_simd<D, WQ, WK, BIAS, WIN>())) void fwd2_kernel(FwdArgs a) {
  using Sh = Fwd2Shape<D, WQ, WK, BIAS>;
  constexpr int BM = Sh::BM, BN = Sh::BN, ND = Sh::ND, NKK = Sh::NKK, NW = Sh::NW, NS = Sh::NS;
  // software pipeline across steps when the ring holds three stages or more
  constexpr bool PIPE = NS >= 3;
  constexpr int LOOK = PIPE ? NS - 2 : NS - 1;  // productions in flight at an acquisition
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  constexpr float kLazy = 8.0f;  // rescale only when a row max grows by > 2^8

  __shared__ __attribute__((aligned(1024))) char smem[Sh::SMEM];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int wq = wave % WQ, wk = wave / WQ;
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_begin = sload1(a.worker_off, worker);
  const int u_end = sload1(a.worker_off, worker + 1);
  const int HD = a.H * D;

  auto stage_k = [&](int s) { return smem + s * Sh::STAGE; };
  auto stage_v = [&](int s) { return smem + s * Sh::STAGE + Sh::K_BYTES; };
  auto stage_b = [&](int s) { return smem + s * Sh::STAGE + Sh::K_BYTES + Sh::V_BYTES; };
  const uint32_t smem_lds = lds_addr(smem);

  // K/V rows permuted only when a bias tile is read (see the header)
  RowLoader<D, 1, BN, NW, BIAS> kload;
  RowLoader<D, 2, BN, NW, BIAS> vload;
  BiasLoader<BN, 1, BM, NW> bload;
  kload.init(wave, lane, HD);
  vload.init(wave, lane, HD);
  static_assert(decltype(kload)::NI == Sh::KNI && decltype(vload)::NI == Sh::VNI &&
                    (!BIAS || decltype(bload)::NI == Sh::BNI),
                "the ring's per-step counts are the loaders' instruction counts");

  // Unit record: sample fields only (three are live at once: producer,
  // current, next); descriptors are rebuilt where they are used.
  struct UnitInfo {
    int b, h, qt, n;
    Sample s;
  };
  auto fetch = [&](int u) {
    UnitInfo x;
    const i32x4 un = sload4(a.units, u);
    x.b = un[0];
    x.h = un[1];
    x.qt = un[2];
    x.n = un[3];
    x.s = sload_sample(a.samples, x.b);
    return x;
  };
  // First element of the unit's (sample, head) bias block.  Derived where it
  // is needed rather than kept in the unit record: state copied between
  // units that a compiler cannot keep in registers lands in scratch, whose
  // accesses wait on vmcnt and with it on the LDS prefetches.
  auto bias_elem0 = [&](const UnitInfo& x) { return x.s.bias0 + (int64_t)x.h * x.s.lq * x.s.lk; };
  // key tile of step t (a windowed unit starts at its window's first tile)
  auto key_tile = [&](const UnitInfo& x, int t) {
    return WIN ? window_first_step(x.qt * BM, a.win_l, BN) + t : t;
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

  // ---- producer: the worker's steps in order, LOOK ahead of the consumer ----
  // Each production moves one step's K and V rows (and bias tile) into a
  // stage.  The descriptors start at the step's first key row and end at the
  // sample end (rows past it read as zero); they are set up once per unit and
  // advanced by a constant per step.
  const int step_ops = loads_of(Sh::KNI, wave, NW) + loads_of(Sh::VNI, wave, NW) + loads_of(Sh::BNI, wave, NW);
  constexpr int MIN_OPS = loads_of(Sh::KNI, NW - 1, NW) + loads_of(Sh::VNI, NW - 1, NW) +
                          loads_of(Sh::BNI, NW - 1, NW);  // the wave with the fewest loads
  constexpr int WAIT_N = (LOOK - 1) * MIN_OPS < 63 ? (LOOK - 1) * MIN_OPS : 63;
  constexpr int32_t KV_STEP = BN * D * 2;  // bytes of one step's rows per head (rows are H heads apart)
  int pu = u_begin, pt = 0, pn = 0, pst = 0;
  Walker<false> wk_k, wk_v;  // K and V rows of the next step
  Walker<true> wk_b;         // bias rows of the next step
  auto start_unit = [&](const UnitInfo& x) {
    const int64_t kvo = ((int64_t)x.s.k0 * a.H + x.h) * D * 2;
    const int64_t row0 = (int64_t)key_tile(x, 0) * BN;
    const int64_t rec = ((int64_t)x.s.lk - row0) * HD * 2;
    wk_k.start(reinterpret_cast<const char*>(a.k) + kvo, row0 * HD * 2, rec);
    wk_v.start(reinterpret_cast<const char*>(a.v) + kvo, row0 * HD * 2, rec);
    if constexpr (BIAS) {
      // rows qt*BM .. of the bias block, keys from row0; the offsets follow lk
      bload.init(wave, lane, x.s.lk);
      const int64_t e0 = bias_elem0(x);
      const int64_t off = ((int64_t)x.qt * BM * x.s.lk + row0) * 2;
      wk_b.start(reinterpret_cast<const char*>(a.bias) + e0 * 2, off, (a.bias_elems - e0) * 2 - off);
    }
  };
  UnitInfo pinfo = fetch(u_begin);
  pn = pinfo.n;
  if (pn > 0) start_unit(pinfo);
  VmLedger<LOOK, WAIT_N> ring;
  auto produce = [&]() {
    if (pt >= pn && pu < u_end) {
      // next unit with steps (units without keys have none)
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
      kload.issue(sb, wk_k.words(), wave);
      vload.issue(sb + Sh::K_BYTES, wk_v.words(), wave);
      if constexpr (BIAS) bload.issue(sb + Sh::K_BYTES + Sh::V_BYTES, wk_b.words(), wave);
      wk_k.advance(KV_STEP * a.H);
      wk_v.advance(KV_STEP * a.H);
      if constexpr (BIAS) wk_b.advance(BN * 2);
      ++pt;
      pst = pst + 1 == NS ? 0 : pst + 1;
      ring.produced(step_ops);
    } else {
      ring.produced(0);
    }
  };
  // the step computed next is the oldest production in flight
  auto acquire = [&]() {
    ring.wait_oldest();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // its tiles are in LDS; every wave is done with the stage produce() refills
    __builtin_amdgcn_sched_barrier(0);
  };

  UnitInfo cur = fetch(u_begin);
  bf16x8 qf[NKK];
  load_q(cur, qf);
  // the first unit's Q has landed before anything else is issued: every later
  // Q load is followed by visible stores, so the compiler's own wait for it
  // at a unit's first step leaves the ring in flight
  wait_vmcnt<0>();
  for (int j = 0; j < LOOK; ++j) produce();
  int stage = 0;  // stage of the step whose softmax comes next

  for (int u = u_begin; u < u_end; ++u) {
    const bool has_next = u + 1 < u_end;
    UnitInfo nxt = cur;
    if (has_next) nxt = fetch(u + 1);
    const int n = cur.n;

    f32x16 oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};
    float m_run = 0.0f, l_run = 0.0f, lr_run = 0.0f;
    bool pad_drop = false;  // this row dropped its padded keys (see the guard below)
    const int kb = wk * 32;  // this wave's key block inside a step

    // S^T of the step in stage st, all MFMAs at once
    auto s_all = [&](int st) {
      const char* kt = stage_k(st);
      f32x16 s = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s = Elem<bf16>::mma(rows_frag<D, 1>(kt, kb + l32, kk, g), qf[kk], s);
      return s;
    };

    // Softmax (or activation) of step t from its scores sacc and the bias
    // tile in stage st: P into pf (and pl), the running max, sums and O
    // rescaled.  FIRST (step 0) starts the running max at the step's max;
    // later steps rescale lazily.  LAST (step n-1) holds the keys past the
    // sample end.  mm(c), c = 0 .. NKK-1, is called between chunks of the
    // exponential (or activation) work, one MFMA of the next step's S^T per
    // call, so that the matrix core runs beside this VALU work; a
    // scheduling fence after each chunk keeps that order.
    auto soft = [&](auto first_tag, auto last_tag, int t, int st, const f32x16& sacc, auto&& mm, bf16x8* pf,
                    bf16x8* pl) {
      constexpr bool FIRST = decltype(first_tag)::value;
      constexpr bool LAST = decltype(last_tag)::value;
      constexpr int PER = 16 / NKK;  // elements of P per interleaved MFMA
      const int key0 = key_tile(cur, t) * BN + kb;  // first key of this wave's block
      // window mask of this wave's 32x32 block (slot keys as described below)
      auto mask = [&](float* v, float fill) {
        const Window w{a.win_l, a.win_r, cur.s.lq, cur.s.lk};
        const int row0 = cur.qt * BM + wq * 32;
        if (!w.full(row0, key0)) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            v[i] = w.allows(row0 + l32, key0 + (BIAS ? 16 * g + i : acc_row(i, g))) ? v[i] : fill;
        }
      };

      // with a bias, slot i of this lane holds key t*BN + kb + 16g + i of
      // query row qt*BM + wq*32 + l32 (else key t*BN + kb + acc_row(i, g))
      float p[16];
      if constexpr (BIAS) {
        const char* bt = stage_b(st) + (wq * 32 + l32) * Sh::BT::PITCH + (kb + 16 * g) * 2;
        bf16x8_to_f32(bt, p);
        bf16x8_to_f32(bt + 16, p + 8);
        if constexpr (LAST) {
          // keys past the sample end carry the next row's bias: they must add
          // nothing (the subtraction below assumes a zero score)
          const int rem = cur.s.lk - (key0 + 16 * g);
#pragma unroll
          for (int i = 0; i < 16; ++i) p[i] = i < rem ? p[i] : 0.0f;
          if (bias_elem0(cur) + (int64_t)cur.s.lq * cur.s.lk == a.bias_elems) {
            // the tensor's last element may straddle the end of the bias
            // range by half a dword, which the range check drops: reload it
            const rsrc_t rl = make_rsrc(reinterpret_cast<const bf16*>(a.bias) + (a.bias_elems - 1), 2);
            const float last = __uint_as_float((uint32_t)buf_load2(rl, 0) << 16);
            const int row = cur.qt * BM + wq * 32 + l32;
#pragma unroll
            for (int i = 0; i < 16; ++i) p[i] = (row == cur.s.lq - 1 && i == rem - 1) ? last : p[i];
          }
        }
      }
      if constexpr (SOFTMAX) {
        // scores in log2 units relative to the running max: x - m
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float c = BIAS ? fmaf(p[i], kLog2e, -m_run) : -m_run;
          p[i] = fmaf(sacc[i], a.scale_log2, c);
        }
        if constexpr (WIN) mask(p, -INFINITY);
        if constexpr (!WIN && LAST) {
          // Guard of the subtraction scheme.  Keys past the sample end score
          // 0 in this last step.  When the row's best valid score is below 0
          // (log2 units), their exp terms would dominate the row sum and the
          // epilogue's subtraction would recover the true sum only through
          // cancellation (or not at all once the valid terms underflow).
          // Such rows drop the padded keys here (p = 0) and skip the
          // subtraction.  The test uses a lower bound of the row's best score
          // (earlier steps reach at least m_run), so it errs towards dropping,
          // which is exact too.
          const int rem = cur.s.lk - key0;  // valid keys of this wave's 32-key block
          if (rem > 0 && rem < 32) {
            float vmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) vmax = (BIAS ? 16 * g + i : acc_row(i, g)) < rem ? fmaxf(vmax, p[i]) : vmax;
            vmax = wave_xor32_max(vmax);
            pad_drop = (FIRST ? vmax : m_run + fmaxf(vmax, 0.0f)) < 0.0f;
            if (pad_drop) {
#pragma unroll
              for (int i = 0; i < 16; ++i) p[i] = (BIAS ? 16 * g + i : acc_row(i, g)) < rem ? p[i] : -INFINITY;
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, p[i]);
        mx = wave_xor32_max(mx);
        if constexpr (FIRST) {
          // the running max starts at this step's max (m_run was 0); with a
          // window the step may hold no visible key of the row
          m_run = WIN ? fmaxf(mx, kNoScore) : mx;
#pragma unroll
          for (int i = 0; i < 16; ++i) p[i] -= m_run;
        } else {
          if (__builtin_amdgcn_ballot_w64(mx > kLazy) != 0) {
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
        }
        // exponentials, row sums and the bf16 operands, interleaved with
        // the next step's MFMAs.  The PV MFMA sees P rounded to bf16; the
        // output is normalised by the sum of exactly those values
        // (v_dot2_f32_bf16 against ones).
        float rs = 0.0f, rsr = 0.0f;
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NKK; ++c) {
          mm(c);
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            const int i = c * PER + j;
            p[i] = fast_exp2(p[i]);
            rs += p[i];
          }
          if ((c + 1) * PER % 8 == 0) {
            const int s8 = (c + 1) * PER / 8 - 1;
            pf[s8] = pack8(&p[s8 * 8]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              rsr = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[s8][2 * j], pf[s8][2 * j + 1]}, ones, rsr, false);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        l_run += rs;
        lr_run += rsr;
      } else {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NKK; ++c) {
          mm(c);
#pragma unroll
          for (int j = 0; j < PER; ++j) {
            const int i = c * PER + j;
            const float x = BIAS ? p[i] + sacc[i] * a.scale : sacc[i] * a.scale;
            p[i] = act_fwd(ACT, x);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (WIN) mask(p, 0.0f);
#pragma unroll
        for (int s8 = 0; s8 < 2; ++s8) {
          pf[s8] = pack8(&p[s8 * 8]);
          if constexpr (SPLIT) {
            float r8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) r8[j] = p[s8 * 8 + j] - (float)pf[s8][j];
            pl[s8] = pack8(r8);
          }
        }
      }
    };

    // O^T += V^T P^T from the V tile in stage st (every V^T read issued
    // before the first MFMA: left to the compiler at this register pressure,
    // the second half of the MFMAs each waits for its own read)
    auto pv = [&](int st, const bf16x8* pf, const bf16x8* pl) {
      const char* vt = stage_v(st);
      bf16x8 va[2][ND];
#pragma unroll
      for (int s8 = 0; s8 < 2; ++s8)
#pragma unroll
        for (int d = 0; d < ND; ++d) va[s8][d] = trans_frag<D, 2>(vt, wk, s8, d * 32, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s8 = 0; s8 < 2; ++s8) {
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const bf16x8 vf = va[s8][d];
          oacc[d] = Elem<bf16>::mma(vf, pf[s8], oacc[d]);
          // split operands matter for the activation path only: softmax
          // already normalises by the sum of the rounded P
          if constexpr (SPLIT && !SOFTMAX) oacc[d] = Elem<bf16>::mma(vf, pl[s8], oacc[d]);
        }
      }
    };
    auto no_mm = [](int) {};
    auto next_stage = [&](int st) { return st + 1 == NS ? 0 : st + 1; };

    if constexpr (PIPE) {
      // Software pipeline: S^T of step t+1 runs on the matrix core while the
      // VALU works on the softmax of step t; then P V of step t.  Two stages
      // are in use at once (t and t+1), so the producer runs NS - 2 ahead.
      // LAST loads the next unit's Q (free once the unit's last S^T is done);
      // it is the only instance that does, so the loop over the other steps
      // carries no register loads in flight and the compiler puts no vmcnt
      // wait of its own into it (such a wait would count only the loads it
      // can see and drain the whole ring).
      auto step = [&](auto first_tag, auto last_tag, int t, f32x16& sacc) {
        constexpr bool LAST = decltype(last_tag)::value;
        bf16x8 pf[2], pl[2];
        if constexpr (LAST) {
          if (has_next) load_q(nxt, qf);
          soft(first_tag, last_tag, t, stage, sacc, no_mm, pf, pl);
        } else {
          acquire();  // step t+1
          produce();
          const char* kn = stage_k(next_stage(stage));
          f32x16 snx = f32x16{};
          bf16x8 ka[NKK];
          constexpr int KA = NKK < 4 ? NKK : 4;  // K fragments in flight
#pragma unroll
          for (int c = 0; c < KA; ++c) ka[c] = rows_frag<D, 1>(kn, kb + l32, c, g);
          auto mm = [&](int c) {
            snx = Elem<bf16>::mma(ka[c], qf[c], snx);
            if (c + KA < NKK) ka[c + KA] = rows_frag<D, 1>(kn, kb + l32, c + KA, g);
          };
          soft(first_tag, last_tag, t, stage, sacc, mm, pf, pl);
          sacc = snx;
        }
        pv(stage, pf, pl);
        stage = next_stage(stage);
      };
      if (n > 0) {
        acquire();  // step 0
        produce();
        f32x16 sacc = s_all(stage);
        if (n == 1) {
          step(std::true_type{}, std::true_type{}, 0, sacc);
        } else {
          step(std::true_type{}, std::false_type{}, 0, sacc);
          for (int t = 1; t + 1 < n; ++t) step(std::false_type{}, std::false_type{}, t, sacc);
          step(std::false_type{}, std::true_type{}, n - 1, sacc);
        }
      }
    } else {
      // one stage in use at a time: acquire, S^T, softmax, P V
      auto step = [&](auto first_tag, auto last_tag, int t) {
        constexpr bool LAST = decltype(last_tag)::value;
        acquire();
        produce();
        const f32x16 sacc = s_all(stage);
        if (LAST && has_next) load_q(nxt, qf);
        bf16x8 pf[2], pl[2];
        soft(first_tag, last_tag, t, stage, sacc, no_mm, pf, pl);
        pv(stage, pf, pl);
        stage = next_stage(stage);
      };
      if (n == 1) {
        step(std::true_type{}, std::true_type{}, 0);
      } else if (n > 1) {
        step(std::true_type{}, std::false_type{}, 0);
        for (int t = 1; t + 1 < n; ++t) step(std::false_type{}, std::false_type{}, t);
        step(std::false_type{}, std::true_type{}, n - 1);
      }
    }
    // ---- epilogue ----
    if constexpr (SOFTMAX) {
      l_run = wave_xor32_sum(l_run);
      lr_run = wave_xor32_sum(lr_run);
      if constexpr (!WIN) {
        // keys past the sample end entered the last step as zeros.  (A window
        // masks them instead; its running max may sit at kNoScore, where
        // 2^-m overflows.)
        int npad = 0;
        if (n > 0 && !pad_drop) npad = 32 - min(max(cur.s.lk - ((n - 1) * BN + wk * 32), 0), 32);
        // (only when there are padded keys: a row without them may sit far
        // below zero, where 2^-m overflows and 0 * inf would be NaN)
        if (npad > 0) {
          const float pad_e = fast_exp2(-m_run);
          l_run -= (float)npad * pad_e;
          lr_run -= (float)npad * (float)(bf16)pad_e;
        }
      }
      if (cur.s.lk <= wk * 32) {
        // this wave's key block lies wholly past the sample end: it holds no
        // term of the row (its O is zero since those V rows read as zero)
        m_run = -INFINITY;
        l_run = 0.0f;
        lr_run = 0.0f;
      }
    }
    const int qrow = cur.qt * BM + wq * 32 + l32;
    const bool valid_row = qrow < cur.s.lq;
    const bool has_keys = cur.s.lk > 0;

    if constexpr (WK > 1) {
      // the stage of the unit's last step (the one before `stage`) is free
      // once every wave passes this barrier: no load refills it before the
      // next acquisition's barrier
      __syncthreads();
      char* free_stage =
          Sh::COMB_IN_STAGE ? smem + (stage == 0 ? NS - 1 : stage - 1) * Sh::STAGE : smem + NS * Sh::STAGE;
      float* ps = reinterpret_cast<float*>(free_stage);
      float* po = reinterpret_cast<float*>(free_stage + Sh::STATS);
      // element (row r of the 32-column block dl of a pass, query l32) of a
      // partial sits at [slot][dl*32 + r][l32]; lane-dependent parts go into one base
      const int lane_off = g * 4 * 32 + l32;
      float fw[WK];  // weight of each key block's partial (block 0 = this wave)
#pragma unroll
      for (int d0 = 0; d0 < ND; d0 += Sh::DP) {
        if (d0 > 0) __syncthreads();  // the previous pass has been read
        if (wk > 0) {
          const int slot = (wk - 1) * WQ + wq;
          float* pw = po + slot * Sh::DP * 32 * 32 + lane_off;
#pragma unroll
          for (int dl = 0; dl < Sh::DP; ++dl)
#pragma unroll
            for (int i = 0; i < 16; ++i) pw[(dl * 32 + (i >> 2) * 8 + (i & 3)) * 32] = oacc[d0 + dl][i];
          if (d0 == 0 && g == 0) {
            ps[(slot * 3 + 0) * 32 + l32] = m_run;
            ps[(slot * 3 + 1) * 32 + l32] = l_run;
            ps[(slot * 3 + 2) * 32 + l32] = lr_run;
          }
        }
        __syncthreads();
        if (wk == 0) {
          if (d0 == 0) {
            float mall = m_run;
            if constexpr (SOFTMAX) {
#pragma unroll
              for (int w2 = 1; w2 < WK; ++w2) mall = fmaxf(mall, ps[(((w2 - 1) * WQ + wq) * 3) * 32 + l32]);
            }
            fw[0] = SOFTMAX ? (has_keys ? fast_exp2(m_run - mall) : 0.0f) : 1.0f;
            float lall = l_run * fw[0], lrall = lr_run * fw[0];
#pragma unroll
            for (int w2 = 1; w2 < WK; ++w2) {
              const int slot = (w2 - 1) * WQ + wq;
              fw[w2] = 1.0f;
              if constexpr (SOFTMAX) {
                fw[w2] = has_keys ? fast_exp2(ps[(slot * 3) * 32 + l32] - mall) : 0.0f;
                lall += ps[(slot * 3 + 1) * 32 + l32] * fw[w2];
                lrall += ps[(slot * 3 + 2) * 32 + l32] * fw[w2];
              }
            }
            m_run = mall;
            l_run = lall;
            lr_run = lrall;
          }
#pragma unroll
          for (int dl = 0; dl < Sh::DP; ++dl) oacc[d0 + dl] *= fw[0];
#pragma unroll
          for (int w2 = 1; w2 < WK; ++w2) {
            const float* pr = po + ((w2 - 1) * WQ + wq) * Sh::DP * 32 * 32 + lane_off;
#pragma unroll
            for (int dl = 0; dl < Sh::DP; ++dl)
#pragma unroll
              for (int i = 0; i < 16; ++i) oacc[d0 + dl][i] += fw[w2] * pr[(dl * 32 + (i >> 2) * 8 + (i & 3)) * 32];
          }
        }
      }
    }

    if (wk == 0) {
      // buffer stores issued by every lane (rows past the sample end at an
      // out-of-range offset), so that the count the ring's waits rely on
      // does not depend on the data; they stay in flight across later waits
      float inv = 1.0f;
      if constexpr (SOFTMAX) inv = has_keys ? 1.0f / lr_run : 0.0f;
      const rsrc_t ro = make_rsrc(reinterpret_cast<const TO*>(a.o) + ((int64_t)cur.s.q0 * a.H + cur.h) * D,
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
        const rsrc_t rl = make_rsrc(a.lse + (int64_t)cur.s.q0 * a.H + cur.h, (uint32_t)cur.s.lq * a.H * 4);
        const float lse = has_keys ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl,
                                              valid_row && g == 0 ? (uint32_t)qrow * a.H * 4 : 0x80000000u, 0, 0);
        ring.counted(1);
      }
    }

    if (has_next && n == 0) {
      // a unit without keys did not load the next Q; waiting here (units
      // without keys are rare) keeps this path from putting a wait that
      // drains the ring into every unit's first step
      load_q(nxt, qf);
      wait_vmcnt<0>();
    }
    cur = nxt;
  }
  // every production was acquired; only stores can still be in flight
  wait_vmcnt<0>();
}

}  // namespace jattn
