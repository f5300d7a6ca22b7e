// dQ kernel of jagged attention for bf16 inputs, gfx950 (dense mask).
//
// Method: "Training GEM at LLM scale" (Meta engineering post), section
// "Jagged Sequence Flash Attention", item "Backward parallelization": dQ has
// its own pass over query tiles, separate from dK/dV, so that no output is
// accumulated with atomic adds.
//
// Workgroup = WQ x WK waves.  A unit is (sample, head, q-tile of 32*WQ rows);
// each K/V step covers BN = 32*WK keys; wave (wq, wk) computes its 32 query
// rows against key block wk of the step:
//     S^T  = K Q^T     A = K rows (LDS),  B = Q fragments (registers)
//     dP^T = V dO^T    A = V rows (LDS),  B = dO fragments (registers)
//     P^T  = exp2(S^T*scale*log2e + bias*log2e - LSE*log2e), one query per lane
//     dS^T = P^T (dP^T - Di)              (or act'(S^T*scale + bias) dP^T)
//     dQ^T += K^T dS^T A = K^T via ds_read_b64_tr_b16, B = dS^T in-register
// K, V and the bias tile travel HBM -> LDS with buffer loads whose
// destination is LDS, double-buffered across steps and units; the key-split
// partials of dQ are summed through LDS at the end of a unit.  K and V rows
// are stored permuted within each 32-key block (RowLoader PERM), so that the
// 16 scores of a lane are 16 consecutive keys and its bias values are two
// aligned 16-byte LDS reads.
//
// Sliding window (WIN, section "BlockAttention"): the unit's steps start at
// the first key tile its window meets; dS is zeroed element-wise in 32x32
// blocks that are not wholly inside the window.
#pragma once
#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace jattn {

template <int D, int WQ, int WK, bool BIAS>
struct Dq2Shape {
  static constexpr int NW = WQ * WK;
  static constexpr int BM = 32 * WQ;  // query rows per unit
  static constexpr int BN = 32 * WK;  // keys per step
  static constexpr int ND = D / 32;
  static constexpr int NKK = D / 16;
  using KT = PadTile<D, 2>;  // K rows, read as rows and transposed
  using VT = PadTile<D, 1>;  // V rows
  static constexpr int K_BYTES = KT::template bytes<BN>();
  static constexpr int V_BYTES = VT::template bytes<BN>();
  using BT = PadTile<BN, 1>;  // bias rows: pitch = 16 (mod 256) bytes, 16-byte reads conflict-free
  static constexpr int B_BYTES = BIAS ? BT::template bytes<BM>() : 0;
  static constexpr int STAGE = K_BYTES + V_BYTES + B_BYTES;
  // dQ^T partials of key blocks 1..WK-1: one pass through a region of their
  // own when the LDS budget allows, else DP 32-column blocks of D per pass
  // through the stage of the unit's last step
  static constexpr int COMB_PER_D = (WK - 1) * WQ * 32 * 32 * 4;
  static constexpr int COMB = COMB_PER_D * ND;
  static constexpr bool COMB_IN_STAGE = WK > 1 && 2 * STAGE + COMB > 160 * 1024;
  static constexpr int DP_FIT = WK > 1 ? STAGE / COMB_PER_D : ND;
  static_assert(!COMB_IN_STAGE || DP_FIT >= 1, "combine pass does not fit a stage");
  static constexpr int DP = !COMB_IN_STAGE || DP_FIT >= ND ? ND : (DP_FIT >= 2 && ND % 2 == 0 ? 2 : 1);
  static constexpr int SMEM = 2 * STAGE + (WK > 1 && !COMB_IN_STAGE ? COMB : 0);
  static_assert(SMEM <= 160 * 1024, "LDS budget");
};

template <typename TG, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT, bool WIN = false>
__global__ __launch_bounds__(64 * WQ * WK, 1) void dq2_kernel(BwdArgs a) {
  using Sh = Dq2Shape<D, WQ, WK, BIAS>;
  constexpr int BM = Sh::BM, BN = Sh::BN, ND = Sh::ND, NKK = Sh::NKK, NW = Sh::NW;
  constexpr bool SOFTMAX = (ACT == kSoftmax);

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
  RowLoader<D, 2, BN, NW, BIAS> kload;
  RowLoader<D, 1, BN, NW, BIAS> vload;
  BiasLoader<BN, 1, BM, NW> bload;
  kload.init(wave, lane, HD);
  vload.init(wave, lane, HD);

  struct UnitInfo {
    int h, qt, n;
    Sample s;
    i32x4 rk, rv;
  };
  auto fetch = [&](int u) {
    UnitInfo x;
    const i32x4 un = load_unit(a.units, u);
    x.h = un[1];
    x.qt = un[2];
    x.n = un[3];
    x.s = load_sample(a.samples, un[0]);
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
  // Q and dO fragments (B operands) and row statistics of this lane's query row
  auto load_q = [&](const UnitInfo& x, bf16x8* qf) {
    const rsrc_t rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + ((int64_t)x.s.q0 * a.H + x.h) * D,
                                (uint32_t)x.s.lq * HD * 2);
    const int row = x.qt * BM + wq * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(row * HD + kk * 16 + g * 8) * 2));
  };
  auto load_do = [&](const UnitInfo& x, bf16x8* dof, float& lse2, float& di) {
    const int64_t qo = ((int64_t)x.s.q0 * a.H + x.h) * D;
    const rsrc_t rdo = make_rsrc(reinterpret_cast<const bf16*>(a.dout) + qo, (uint32_t)x.s.lq * HD * 2);
    const int row = x.qt * BM + wq * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      dof[kk] = __builtin_bit_cast(bf16x8, buf_load16(rdo, (uint32_t)(row * HD + kk * 16 + g * 8) * 2));
    if constexpr (SOFTMAX) {
      // rows past the sample end read as zero, which keeps their terms finite
      const uint32_t rec = (uint32_t)x.s.lq * a.H * 4;
      const rsrc_t rl = make_rsrc(a.lse2 + (int64_t)x.s.q0 * a.H + x.h, rec);
      const rsrc_t rd = make_rsrc(a.di + (int64_t)x.s.q0 * a.H + x.h, rec);
      lse2 = __uint_as_float(buf_load4(rl, (uint32_t)row * a.H * 4));
      di = __uint_as_float(buf_load4(rd, (uint32_t)row * a.H * 4));
    }
  };

  if (u_begin >= u_end) return;
  UnitInfo cur = fetch(u_begin);
  bf16x8 qf[NKK], dof[NKK];
  float lse2 = 0.0f, di = 0.0f;
  load_q(cur, qf);
  load_do(cur, dof, lse2, di);
  int stage = 0;
  if (cur.n > 0) issue_step(cur, 0, 0);

  for (int u = u_begin; u < u_end; ++u) {
    const bool has_next = u + 1 < u_end;
    UnitInfo nxt = cur;
    if (has_next) nxt = fetch(u + 1);
    const int n = cur.n;
    // row statistics of this unit (the next unit's are loaded during its last step)
    const float lse2_u = lse2, di_u = di;

    f32x16 dqacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) dqacc[d] = f32x16{};

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
      const int key0 = key_tile(cur, t) * BN + kb;  // its first key

      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      {
        bf16x8 ka[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) ka[kk] = rows_frag<D, 2>(kt, kb + l32, kk, g);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) sacc = Elem<bf16>::mma(ka[kk], qf[kk], sacc);
      }
      if (t + 1 == n && has_next) load_q(nxt, qf);
      {
        bf16x8 va[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) va[kk] = rows_frag<D, 1>(vt, kb + l32, kk, g);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) dpacc = Elem<bf16>::mma(va[kk], dof[kk], dpacc);
      }
      if (t + 1 == n && has_next) load_do(nxt, dof, lse2, di);

      // with a bias, slot i of this lane holds key t*BN + kb + 16g + i of
      // query row qt*BM + wq*32 + l32 (else key t*BN + kb + acc_row(i, g))
      float ds[16];
      const int rem = cur.s.lk - (key0 + (BIAS ? 16 * g : 0));  // keys >= lk: slot key >= rem
      if constexpr (BIAS) {
        const char* bt = stage_b(stage) + (wq * 32 + l32) * Sh::BT::PITCH + (kb + 16 * g) * 2;
        bf16x8_to_f32(bt, ds);
        bf16x8_to_f32(bt + 16, ds + 8);
        if (t + 1 == n && bias_elem0(cur) + (int64_t)cur.s.lq * cur.s.lk == a.bias_elems) {
          // the tensor's last element may straddle the end of the bias range
          // by half a dword, which the range check drops: reload it
          const rsrc_t rl = make_rsrc(reinterpret_cast<const bf16*>(a.bias) + (a.bias_elems - 1), 2);
          const float last = __uint_as_float((uint32_t)buf_load2(rl, 0) << 16);
          const int row = cur.qt * BM + wq * 32 + l32;
#pragma unroll
          for (int i = 0; i < 16; ++i) ds[i] = (row == cur.s.lq - 1 && i == rem - 1) ? last : ds[i];
        }
      }
      if constexpr (SOFTMAX) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float c = BIAS ? fmaf(ds[i], kLog2e, -lse2_u) : -lse2_u;
          const float p = fast_exp2(fmaf(sacc[i], a.scale_log2, c));
          ds[i] = p * (dpacc[i] - di_u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = BIAS ? fmaf(sacc[i], a.scale, ds[i]) : sacc[i] * a.scale;
          ds[i] = act_grad(ACT, x) * dpacc[i];
        }
      }
      if constexpr (WIN) {
        // pairs outside the window and keys past the sample end add nothing
        const Window w{a.win_l, a.win_r, cur.s.lq, cur.s.lk};
        const int row0 = cur.qt * BM + wq * 32;
        if (!w.full(row0, key0)) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            ds[i] = w.allows(row0 + l32, key0 + (BIAS ? 16 * g + i : acc_row(i, g))) ? ds[i] : 0.0f;
        }
      } else if (t + 1 == n) {
        // keys past the sample end (zero K/V rows, bias of the next row): their
        // dS must be exactly zero, whatever P overflowed to
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = (BIAS ? i : acc_row(i, g)) < rem ? ds[i] : 0.0f;
      }

#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 dh = pack8(&ds[st * 8]);
        bf16x8 dl;
        if constexpr (SPLIT) {
          float r8[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) r8[j] = ds[st * 8 + j] - (float)dh[j];
          dl = pack8(r8);
        }
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const bf16x8 kf = trans_frag<D, 2>(kt, wk, st, d * 32, lane);
          dqacc[d] = Elem<bf16>::mma(kf, dh, dqacc[d]);
          if constexpr (SPLIT) dqacc[d] = Elem<bf16>::mma(kf, dl, dqacc[d]);
        }
      }
      stage ^= 1;
    }

    // ---- epilogue: sum the key-block partials, dQ = scale * dQ^T^T ----
    const int qrow = cur.qt * BM + wq * 32 + l32;
    TG* qrp = reinterpret_cast<TG*>(a.dq) + ((int64_t)(cur.s.q0 + qrow) * a.H + cur.h) * D;
    if constexpr (WK > 1) {
      if (n > 0) {
        // the stage of the last step is free once every wave passes this barrier
        __syncthreads();
        float* po = reinterpret_cast<float*>(Sh::COMB_IN_STAGE ? smem + (stage ^ 1) * Sh::STAGE
                                                               : smem + 2 * Sh::STAGE);
        const int lane_off = g * 4 * 32 + l32;
#pragma unroll
        for (int d0 = 0; d0 < ND; d0 += Sh::DP) {
          if (d0 > 0) __syncthreads();  // the previous pass has been read
          if (wk > 0) {
            float* pw = po + ((wk - 1) * WQ + wq) * Sh::DP * 32 * 32 + lane_off;
#pragma unroll
            for (int dl = 0; dl < Sh::DP; ++dl)
#pragma unroll
              for (int i = 0; i < 16; ++i) pw[(dl * 32 + (i >> 2) * 8 + (i & 3)) * 32] = dqacc[d0 + dl][i];
          }
          __syncthreads();
          if (wk == 0) {
#pragma unroll
            for (int w2 = 1; w2 < WK; ++w2) {
              const float* pr = po + ((w2 - 1) * WQ + wq) * Sh::DP * 32 * 32 + lane_off;
#pragma unroll
              for (int dl = 0; dl < Sh::DP; ++dl)
#pragma unroll
                for (int i = 0; i < 16; ++i) dqacc[d0 + dl][i] += pr[(dl * 32 + (i >> 2) * 8 + (i & 3)) * 32];
            }
          }
        }
      }
    }
    if (wk == 0 && qrow < cur.s.lq) {
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          store4<TG>(qrp + d * 32 + i4 * 8 + g * 4, dqacc[d][i4 * 4] * a.scale, dqacc[d][i4 * 4 + 1] * a.scale,
                     dqacc[d][i4 * 4 + 2] * a.scale, dqacc[d][i4 * 4 + 3] * a.scale);
    }

    if (has_next) {
      if (n == 0) {
        // a unit without keys issued no prefetch
        load_q(nxt, qf);
        load_do(nxt, dof, lse2, di);
      }
      if (n == 0 && nxt.n > 0) {
        wait_vmcnt0();
        __syncthreads();
        issue_step(nxt, 0, stage);
      }
    }
    cur = nxt;
  }
}

}  // namespace jattn
