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
// destination is LDS into a ring of NS stages: a producer cursor runs NS - 1
// steps ahead of the step being computed, across unit boundaries, and each
// step waits only for its own loads (exact per-wave counts, dQ stores
// included).  The key-split partials of dQ are summed through LDS at the end
// of a unit.  K and V rows
// are stored permuted within each 32-key block (RowLoader PERM), so that the
// 16 scores of a lane are 16 consecutive keys and its bias values are two
// aligned 16-byte LDS reads.
//
// Sliding window (WIN, section "BlockAttention"): the unit's steps start at
// the first key tile its window meets; dS is zeroed element-wise in 32x32
// blocks that are not wholly inside the window.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"
#include "ring.hpp"

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
  // ring depth: up to four stages (three steps in flight beside the one computed)
  static constexpr int NS_FIT = 160 * 1024 / STAGE;
  static constexpr int NS = NS_FIT >= 4 ? 4 : NS_FIT;
  static_assert(NS >= 2, "two stages at least");
  // LDS-destination load instructions of one step (whole workgroup)
  static constexpr int KNI = KT::template ninst<BN>();
  static constexpr int VNI = VT::template ninst<BN>();
  static constexpr int BNI = BIAS ? BT::template ninst<BM>() : 0;
  // dQ^T partials of key blocks 1..WK-1: one pass through a region of their
  // own when the LDS budget allows, else DP 32-column blocks of D per pass
  // through the stage of the unit's last step
  static constexpr int COMB_PER_D = (WK - 1) * WQ * 32 * 32 * 4;
  static constexpr int COMB = COMB_PER_D * ND;
  static constexpr bool COMB_IN_STAGE = WK > 1 && NS * STAGE + COMB > 160 * 1024;
  static constexpr int DP_FIT = WK > 1 ? STAGE / COMB_PER_D : ND;
  static_assert(!COMB_IN_STAGE || DP_FIT >= 1, "combine pass does not fit a stage");
  static constexpr int DP = !COMB_IN_STAGE || DP_FIT >= ND ? ND : (DP_FIT >= 2 && ND % 2 == 0 ? 2 : 1);
  static constexpr int SMEM = NS * STAGE + (WK > 1 && !COMB_IN_STAGE ? COMB : 0);
  static_assert(SMEM <= 160 * 1024, "LDS budget");
};

// 4 query groups x one key block without a bias or window run two
// workgroups per CU (the plan gives that shape twice the workers; three at
// D = 64 would spill the bf16-gradient instance that reads fp32 O); the
// other shapes keep the default (at least one)
template <int D, int WQ, int WK, bool BIAS, bool WIN>
constexpr int dq2_waves_per_simd() {
  return WQ == 4 && WK == 1 && !BIAS && !WIN ? 2 : 1;
}

// OF (softmax only): 0 = Di and LSE*log2e read from the workspace; 1 / 2 =
// formed here from O (bf16 / fp32), dO and the natural LSE, and written to
// the workspace for the dK/dV pass, which then runs after this one.
template <typename TG, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT, bool WIN = false, int OF = 0>
__global__ __launch_bounds__(64 * WQ * WK, (dq2_waves_per_simd<D, WQ, WK, BIAS, WIN>())) void dq2_kernel(BwdArgs a) {
  using Sh = Dq2Shape<D, WQ, WK, BIAS>;
  constexpr int BM = Sh::BM, BN = Sh::BN, ND = Sh::ND, NKK = Sh::NKK, NW = Sh::NW, NS = Sh::NS;
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  constexpr bool FOLD = SOFTMAX && OF != 0;
  static_assert(OF == 0 || SOFTMAX, "row statistics belong to softmax");

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
  RowLoader<D, 2, BN, NW, BIAS> kload;
  RowLoader<D, 1, BN, NW, BIAS> vload;
  BiasLoader<BN, 1, BM, NW> bload;
  kload.init(wave, lane, HD);
  vload.init(wave, lane, HD);
  static_assert(decltype(kload)::NI == Sh::KNI && decltype(vload)::NI == Sh::VNI &&
                    (!BIAS || decltype(bload)::NI == Sh::BNI),
                "the ring's per-step counts are the loaders' instruction counts");

  // Unit record: sample fields only (three are live at once: producer,
  // current, next); descriptors are rebuilt where they are used.
  struct UnitInfo {
    int h, qt, n;
    Sample s;
  };
  auto fetch = [&](int u) {
    UnitInfo x;
    const i32x4 un = sload4(a.units, u);
    x.h = un[1];
    x.qt = un[2];
    x.n = un[3];
    x.s = sload_sample(a.samples, un[0]);
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
  // Q and dO fragments (B operands) and row statistics of this lane's query row
  auto load_q = [&](const UnitInfo& x, bf16x8* qf) {
    const rsrc_t rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + ((int64_t)x.s.q0 * a.H + x.h) * D,
                                (uint32_t)x.s.lq * HD * 2);
    const int row = x.qt * BM + wq * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(row * HD + kk * 16 + g * 8) * 2));
  };
  // O of this lane's row in the dO layout (FOLD: bf16 or fp32 elements)
  bf16x8 o16[OF == 1 ? NKK : 1];
  f32x4 o32[OF == 2 ? 2 * NKK : 1];
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
      if constexpr (FOLD) {
        // O and the natural LSE; Di and LSE*log2e are formed at the unit's start
        if constexpr (OF == 1) {
          const rsrc_t ro = make_rsrc(reinterpret_cast<const bf16*>(a.o) + qo, (uint32_t)x.s.lq * HD * 2);
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk)
            o16[kk] = __builtin_bit_cast(bf16x8, buf_load16(ro, (uint32_t)(row * HD + kk * 16 + g * 8) * 2));
        } else {
          const rsrc_t ro = make_rsrc(reinterpret_cast<const float*>(a.o) + qo, (uint32_t)x.s.lq * HD * 4);
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            o32[2 * kk] = __builtin_bit_cast(f32x4, buf_load16(ro, (uint32_t)(row * HD + kk * 16 + g * 8) * 4));
            o32[2 * kk + 1] = __builtin_bit_cast(f32x4, buf_load16(ro, (uint32_t)(row * HD + kk * 16 + g * 8 + 4) * 4));
          }
        }
        lse2 = __uint_as_float(buf_load4(make_rsrc(a.lse + (int64_t)x.s.q0 * a.H + x.h, rec), (uint32_t)row * a.H * 4));
      } else {
        const rsrc_t rl = make_rsrc(a.lse2 + (int64_t)x.s.q0 * a.H + x.h, rec);
        const rsrc_t rd = make_rsrc(a.di + (int64_t)x.s.q0 * a.H + x.h, rec);
        lse2 = __uint_as_float(buf_load4(rl, (uint32_t)row * a.H * 4));
        di = __uint_as_float(buf_load4(rd, (uint32_t)row * a.H * 4));
      }
    }
  };

  if (u_begin >= u_end) return;

  // ---- producer: the worker's steps in order, NS - 1 ahead of the consumer ----
  // Each production moves one step's K and V rows (and bias tile) into a
  // stage.  The descriptors start at the step's first key row and end at the
  // sample end (rows past it read as zero); they are set up once per unit and
  // advanced by a constant per step.
  constexpr int LOOK = NS - 1;  // productions in flight at an acquisition
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

  UnitInfo cur = fetch(u_begin);
  bf16x8 qf[NKK], dof[NKK];
  float lse2 = 0.0f, di = 0.0f;
  load_q(cur, qf);
  load_do(cur, dof, lse2, di);
  // the first unit's rows have landed before anything else is issued: every
  // later row load is followed by visible stores, so the compiler's own wait
  // for them at a unit's first step leaves the ring in flight
  wait_vmcnt<0>();
  for (int j = 0; j < LOOK; ++j) produce();
  int stage = 0;  // stage of the step computed next

  for (int u = u_begin; u < u_end; ++u) {
    const bool has_next = u + 1 < u_end;
    UnitInfo nxt = cur;
    if (has_next) nxt = fetch(u + 1);
    const int n = cur.n;
    // row statistics of this unit (the next unit's rows are loaded during its last step)
    float lse2_u = lse2, di_u = di;
    if constexpr (FOLD) {
      // Di = rowsum(dO * O) (each lane half holds half of the row) and
      // LSE * log2(e), written for the dK/dV pass by the waves of key block 0
      // (buffer stores from every lane, counted like the dQ stores)
      float part = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if constexpr (OF == 1) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            part = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{dof[kk][2 * j], dof[kk][2 * j + 1]},
                                                   bf16x2{o16[kk][2 * j], o16[kk][2 * j + 1]}, part, false);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) part = fmaf((float)dof[kk][j], o32[2 * kk + j / 4][j % 4], part);
        }
      }
      di_u = wave_xor32_sum(part);
      lse2_u = lse2 * kLog2e;
      if (wk == 0) {
        const int row = cur.qt * BM + wq * 32 + l32;
        const uint32_t rec = (uint32_t)cur.s.lq * a.H * 4;
        const uint32_t voff = row < cur.s.lq && g == 0 ? (uint32_t)row * a.H * 4 : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(di_u), make_rsrc(a.rs_di + (int64_t)cur.s.q0 * a.H + cur.h, rec),
                                              voff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse2_u),
                                              make_rsrc(a.rs_lse2 + (int64_t)cur.s.q0 * a.H + cur.h, rec), voff, 0, 0);
        ring.counted(2);
      }
    }

    f32x16 dqacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) dqacc[d] = f32x16{};

    // LAST (step n-1) loads the next unit's rows; it is the only instance
    // that does, so the loop over the other steps carries no register loads
    // in flight and the compiler puts no vmcnt wait of its own into it (such
    // a wait would count only the loads it can see and drain the whole ring).
    auto step = [&](auto last_tag, int t) {
      constexpr bool LAST = decltype(last_tag)::value;
      // step t is the oldest production in flight: wait for its loads only
      ring.wait_oldest();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // its tiles are in LDS; every wave is done with the stage produce() refills
      __builtin_amdgcn_sched_barrier(0);
      produce();
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
      if (LAST && has_next) load_q(nxt, qf);
      {
        bf16x8 va[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) va[kk] = rows_frag<D, 1>(vt, kb + l32, kk, g);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) dpacc = Elem<bf16>::mma(va[kk], dof[kk], dpacc);
      }
      if (LAST && has_next) load_do(nxt, dof, lse2, di);

      // with a bias, slot i of this lane holds key t*BN + kb + 16g + i of
      // query row qt*BM + wq*32 + l32 (else key t*BN + kb + acc_row(i, g))
      float ds[16];
      const int rem = cur.s.lk - (key0 + (BIAS ? 16 * g : 0));  // keys >= lk: slot key >= rem
      if constexpr (BIAS) {
        const char* bt = stage_b(stage) + (wq * 32 + l32) * Sh::BT::PITCH + (kb + 16 * g) * 2;
        bf16x8_to_f32(bt, ds);
        bf16x8_to_f32(bt + 16, ds + 8);
        if (LAST && bias_elem0(cur) + (int64_t)cur.s.lq * cur.s.lk == a.bias_elems) {
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
      } else if (LAST) {
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
      stage = stage + 1 == NS ? 0 : stage + 1;
    };
    if (n > 0) {
      for (int t = 0; t + 1 < n; ++t) step(std::false_type{}, t);
      step(std::true_type{}, n - 1);
    }

    // ---- epilogue: sum the key-block partials, dQ = scale * dQ^T^T ----
    const int qrow = cur.qt * BM + wq * 32 + l32;
    if constexpr (WK > 1) {
      if (n > 0) {
        // the stage of the unit's last step (the one before `stage`) is free
        // once every wave passes this barrier: no load refills it before the
        // next acquisition's barrier
        __syncthreads();
        float* po = reinterpret_cast<float*>(
            Sh::COMB_IN_STAGE ? smem + (stage == 0 ? NS - 1 : stage - 1) * Sh::STAGE : smem + NS * Sh::STAGE);
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
    if (wk == 0) {
      // buffer stores issued by every lane (rows past the sample end at an
      // out-of-range offset), so that the count the ring's waits rely on
      // does not depend on the data; they stay in flight across later waits
      const rsrc_t rq = make_rsrc(reinterpret_cast<const TG*>(a.dq) + ((int64_t)cur.s.q0 * a.H + cur.h) * D,
                                  (uint32_t)cur.s.lq * HD * (uint32_t)sizeof(TG));
      const uint32_t vrow = qrow < cur.s.lq ? (uint32_t)(qrow * HD) * (uint32_t)sizeof(TG) : 0x80000000u;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          buf_store4<TG>(rq, vrow + (uint32_t)(d * 32 + i4 * 8 + g * 4) * (uint32_t)sizeof(TG),
                         dqacc[d][i4 * 4] * a.scale, dqacc[d][i4 * 4 + 1] * a.scale, dqacc[d][i4 * 4 + 2] * a.scale,
                         dqacc[d][i4 * 4 + 3] * a.scale);
      ring.counted(ND * 4);
    }

    if (has_next && n == 0) {
      // a unit without keys did not load the next unit's rows; waiting here
      // (units without keys are rare) keeps this path from putting a wait
      // that drains the ring into every unit's first step
      load_q(nxt, qf);
      load_do(nxt, dof, lse2, di);
      wait_vmcnt<0>();
    }
    cur = nxt;
  }
  // every production was acquired; only stores can still be in flight
  wait_vmcnt<0>();
}

}  // namespace jattn
