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
// while step t computes; one barrier per step.  K and V rows are stored
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
  static constexpr bool COMB_IN_STAGE = WK > 1 && 2 * STAGE + OWN > 160 * 1024;
  static_assert(!COMB_IN_STAGE || DP_FIT >= 1, "combine pass does not fit a stage");
  static constexpr int DP = !COMB_IN_STAGE || DP_FIT >= ND ? ND : (DP_FIT >= 2 && ND % 2 == 0 ? 2 : 1);
  static constexpr int EXTRA = (WK > 1 && !COMB_IN_STAGE) ? OWN : 0;
  static constexpr int SMEM = 2 * STAGE + EXTRA;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
};

template <typename TO, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT, bool WIN = false>
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

  // K/V rows permuted only when a bias tile is read (see the header)
  RowLoader<D, 1, BN, NW, BIAS> kload;
  RowLoader<D, 2, BN, NW, BIAS> vload;
  BiasLoader<BN, 1, BM, NW> bload;
  kload.init(wave, lane, HD);
  vload.init(wave, lane, HD);

  struct UnitInfo {
    int b, h, qt, n;
    Sample s;
    i32x4 rk, rv;  // descriptors at row 0 of this (sample, head)
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
  // issue the HBM -> LDS loads of step t of unit x into stage st: the K and V
  // descriptors start at the step's first key row and end at the sample end
  auto issue_step = [&](const UnitInfo& x, int t, int st) {
    const uint32_t sb = smem_lds + st * Sh::STAGE;
    const int kt = key_tile(x, t);
    const int64_t row0 = (int64_t)kt * BN;
    const int64_t rec = (int64_t)(x.s.lk - kt * BN) * HD * 2;
    kload.issue(sb, rsrc_at(x.rk, row0 * HD * 2, rec), wave);
    vload.issue(sb + Sh::K_BYTES, rsrc_at(x.rv, row0 * HD * 2, rec), wave);
    if constexpr (BIAS) {
      // rows qt*BM .. of the bias block, keys t*BN ..; the offsets follow lk
      if (t == 0) bload.init(wave, lane, x.s.lk);
      const int64_t e0 = bias_elem0(x);
      const int64_t off = ((int64_t)x.qt * BM * x.s.lk + row0) * 2;
      const i32x4 rb = rsrc_words(reinterpret_cast<const bf16*>(a.bias) + e0, 0);
      bload.issue(sb + Sh::K_BYTES + Sh::V_BYTES, rsrc_at(rb, off, (a.bias_elems - e0) * 2 - off), wave);
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
    bool pad_drop = false;  // this row dropped its padded keys (see the guard below)

    // One K/V step.  FIRST (step 0) starts the running max at the step's
    // max; later steps rescale lazily.  Separate instances keep the
    // accumulators in place across the rescale branch.
    auto step = [&](auto first_tag, int t) {
      constexpr bool FIRST = decltype(first_tag)::value;
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
      const int key0 = key_tile(cur, t) * BN + kb;  // its first key
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

      f32x16 sacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) sacc = Elem<bf16>::mma(rows_frag<D, 1>(kt, kb + l32, kk, g), qf[kk], sacc);
      // Q is dead after the last S^T of the unit: fetch the next unit's rows
      if (t + 1 == n && has_next) load_q(nxt, qf);

      // with a bias, slot i of this lane holds key t*BN + kb + 16g + i of
      // query row qt*BM + wq*32 + l32 (else key t*BN + kb + acc_row(i, g))
      float p[16];
      if constexpr (BIAS) {
        const char* bt = stage_b(stage) + (wq * 32 + l32) * Sh::BT::PITCH + (kb + 16 * g) * 2;
        bf16x8_to_f32(bt, p);
        bf16x8_to_f32(bt + 16, p + 8);
        if (t + 1 == n) {
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
      bf16x8 pf[2], pl[2];
      if constexpr (SOFTMAX) {
        // scores in log2 units relative to the running max: x - m
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float c = BIAS ? fmaf(p[i], kLog2e, -m_run) : -m_run;
          p[i] = fmaf(sacc[i], a.scale_log2, c);
        }
        if constexpr (WIN) mask(p, -INFINITY);
        if constexpr (!WIN) {
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
          if (t + 1 == n && rem > 0 && rem < 32) {
            float vm = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) vm = (BIAS ? 16 * g + i : acc_row(i, g)) < rem ? fmaxf(vm, p[i]) : vm;
            vm = wave_xor32_max(vm);
            pad_drop = (FIRST ? vm : m_run + fmaxf(vm, 0.0f)) < 0.0f;
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
        if constexpr (WIN) mask(p, 0.0f);
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
    };
    if (n > 0) {
      step(std::true_type{}, 0);
      for (int t = 1; t < n; ++t) step(std::false_type{}, t);
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
    TO* orow = reinterpret_cast<TO*>(a.o) + ((int64_t)(cur.s.q0 + qrow) * a.H + cur.h) * D;
    const bool valid_row = qrow < cur.s.lq;
    const bool has_keys = cur.s.lk > 0;

    if constexpr (WK > 1) {
      // stage that held the last step is free once every wave passes this barrier
      __syncthreads();
      char* free_stage = Sh::COMB_IN_STAGE ? smem + (stage ^ 1) * Sh::STAGE : smem + 2 * Sh::STAGE;
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
