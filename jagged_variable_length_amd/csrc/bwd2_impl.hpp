// dK/dV kernel of jagged attention for bf16 inputs, gfx950 (dense mask).
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
// Memory pipeline: Q, dO, the bias tile and the row statistics of a step go
// HBM -> LDS with buffer loads whose destination is LDS, NS steps deep (a
// ring of stages; step c + NS - 1 is issued while step c computes, also
// across unit boundaries).  K and V of a unit live in registers; the next
// unit's K/V are loaded during the last step of the current unit, right
// after their last use.  Each wait counts only the loads issued after the data it
// needs (loads return in order), so the prefetches stay in flight.
#pragma once
#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace jattn {

// Plan records through scalar loads: addresses are wave-uniform and the data
// is read-only for the whole launch, so the constant address space applies.
// Scalar loads are counted by lgkmcnt, which keeps the compiler from placing
// vmcnt waits (and with them waits on the LDS prefetches) on plan reads.
typedef __attribute__((address_space(4))) const int32_t c_i32;
typedef __attribute__((address_space(4))) const i32x4 c_i32x4;

__device__ __forceinline__ int sload1(const int32_t* p, int i) { return ((c_i32*)p)[i]; }
__device__ __forceinline__ i32x4 sload4(const int32_t* p, int i) { return ((c_i32x4*)p)[i]; }

__device__ __forceinline__ Sample sload_sample(const int32_t* table, int b) {
  const i32x4 x = sload4(table, 2 * b);
  const i32x4 y = sload4(table, 2 * b + 1);
  Sample s;
  s.q0 = x[0];
  s.lq = x[1];
  s.k0 = x[2];
  s.lk = x[3];
  s.bias0 = (int64_t)(uint32_t)y[0] | ((int64_t)y[1] << 32);
  return s;
}

// s_waitcnt vmcnt(n), n <= 63 (expcnt and lgkmcnt at their maximum)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// 16-byte register load issued as inline asm: the compiler does not track it,
// the kernel waits for it explicitly (see the unit switch below).
__device__ __forceinline__ void asm_load16(bf16x8& dst, const i32x4& r, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(dst) : "v"(voff), "s"(r) : "memory");
}

template <int D, int WKV, int WKQ, bool SOFTMAX, bool BIAS>
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
  static constexpr int NS_FIT = 160 * 1024 / STAGE;
  static constexpr int NS = NS_FIT >= 3 ? 3 : 2;
  static constexpr int SMEM = NS * STAGE;
  // loads that every wave issues per step (the minimum over waves)
  static constexpr int QNI = QT::template ninst<QS>();
  static constexpr int L_MIN =
      2 * (QNI / NW) + (BIAS ? BT::template ninst<QS>() / NW : 0) + (NRS >= NW ? NRS / NW : 0);
  static_assert(NS_FIT >= 2 && COMB <= STAGE, "LDS budget");
  static_assert(NW == 4, "four waves");
  static_assert(L_MIN < 64, "vmcnt range");
};

// DBIAS: 0 = no dBias, 1 = bf16 dBias, 2 = fp32 dBias
template <typename TG, int D, int WKV, int WKQ, int ACT, bool BIAS, int DBIAS, bool SPLIT>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void dkdv2_kernel(BwdArgs a) {
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  using Sh = Dkdv2Shape<D, WKV, WKQ, SOFTMAX, BIAS>;
  constexpr int NW = Sh::NW, KT = Sh::KT, QS = Sh::QS, ND = D / 32, NKK = D / 16, NS = Sh::NS;
  constexpr int PAD = Sh::PAD, L = Sh::L_MIN;
  constexpr int ESB = DBIAS == 2 ? 4 : 2;  // dBias element size

  __shared__ __attribute__((aligned(1024))) char smem[Sh::SMEM];
  const uint32_t smem_lds = lds_addr(smem);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int wv = wave % WKV, wq = wave / WKV;
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_begin = sload1(a.worker_off, worker);
  const int u_end = sload1(a.worker_off, worker + 1);
  const int H = a.H, HD = a.H * D;

  RowLoader<D, PAD, QS, NW> qload;
  BiasLoader<KT, 1, QS, NW> bload;
  qload.init(wave, lane, HD);
  const uint32_t rs_voff = (uint32_t)lane * H * 4;  // row-stat load: lane l -> query row l of the load

  struct Unit {
    int h, kt, n;
    Sample s;
    i32x4 rq, rdo, rl, rd, rb;  // descriptors at query row 0 of the (sample, head)
    int64_t brec;               // bytes from the bias block start to the end of the bias tensor
    bool tail;                  // the bias block holds the tensor's last element
  };
  auto fetch = [&](int u) {
    Unit x{};
    const i32x4 un = sload4(a.units, u);
    x.h = un[1];
    x.kt = un[2];
    x.n = un[3];
    x.s = sload_sample(a.samples, un[0]);
    const int64_t qo = ((int64_t)x.s.q0 * H + x.h) * D;
    x.rq = rsrc_words(reinterpret_cast<const bf16*>(a.q) + qo, 0);
    x.rdo = rsrc_words(reinterpret_cast<const bf16*>(a.dout) + qo, 0);
    if constexpr (SOFTMAX) {
      x.rl = rsrc_words(a.lse2 + (int64_t)x.s.q0 * H + x.h, 0);
      x.rd = rsrc_words(a.di + (int64_t)x.s.q0 * H + x.h, 0);
    }
    if constexpr (BIAS) {
      const int64_t e0 = x.s.bias0 + (int64_t)x.h * x.s.lq * x.s.lk;
      x.rb = rsrc_words(reinterpret_cast<const bf16*>(a.bias) + e0, 0);
      x.brec = (a.bias_elems - e0) * 2;
      x.tail = e0 + (int64_t)x.s.lq * x.s.lk == a.bias_elems;
    }
    return x;
  };

  // ---- producer: HBM -> LDS loads of one step into one stage ----
  auto issue_step = [&](const Unit& x, int t, int st) {
    const uint32_t sb = smem_lds + st * Sh::STAGE;
    const int r0 = t * QS;
    const int64_t rec = (int64_t)(x.s.lq - r0) * HD * 2;
    qload.issue(sb, rsrc_at(x.rq, (int64_t)r0 * HD * 2, rec), wave);
    qload.issue(sb + Sh::OFF_O, rsrc_at(x.rdo, (int64_t)r0 * HD * 2, rec), wave);
    if constexpr (SOFTMAX) {
      // load j: rows 64*(j % (NRS/2)) .. of LSE (j < NRS/2) or Di
      constexpr int HALF = Sh::NRS / 2;
#pragma unroll
      for (int j = 0; j < Sh::NRS; j += NW) {
        const int jj = j + wave;
        if (jj < Sh::NRS) {
          const int rr = r0 + 64 * (jj % HALF);
          const i32x4 base = jj < HALF ? x.rl : x.rd;
          const uint32_t voff = 64 * (jj % HALF) + lane < QS ? rs_voff : 0x80000000u;
          lds_dma4(rsrc_at(base, (int64_t)rr * H * 4, (int64_t)(x.s.lq - rr) * H * 4),
                   sb + Sh::OFF_RS + jj * 256, voff);
        }
      }
    }
    if constexpr (BIAS) {
      // query rows t*QS .., keys kt*KT .. of the bias block; the offsets follow lk
      if (t == 0) bload.init(wave, lane, x.s.lk);
      const int64_t off = ((int64_t)r0 * x.s.lk + (int64_t)x.kt * KT) * 2;
      bload.issue(sb + Sh::OFF_B, rsrc_at(x.rb, off, x.brec - off), wave);
    }
  };

  // producer cursor: next (unit, step) to issue; units without steps are skipped
  int pu = u_begin, pt = 0, pst = 0;
  Unit pinfo;
  if (pu < u_end) pinfo = fetch(pu);
  auto produce = [&]() -> bool {
    while (pu < u_end && pt >= pinfo.n) {
      ++pu;
      pt = 0;
      if (pu < u_end) pinfo = fetch(pu);
    }
    if (pu >= u_end) return false;
    issue_step(pinfo, pt, pst);
    ++pt;
    pst = pst + 1 == NS ? 0 : pst + 1;
    return true;
  };

  // K and V fragments (MFMA B operand) of this lane's key row
  auto load_kv = [&](const Unit& x, bf16x8* kf, bf16x8* vf) {
    const int64_t ko = ((int64_t)x.s.k0 * H + x.h) * D;
    const uint32_t rec = (uint32_t)x.s.lk * HD * 2;
    const i32x4 rk = rsrc_words(reinterpret_cast<const bf16*>(a.k) + ko, rec);
    const i32x4 rv = rsrc_words(reinterpret_cast<const bf16*>(a.v) + ko, rec);
    const int key = x.kt * KT + wv * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint32_t voff = (uint32_t)(key * HD + kk * 16 + g * 8) * 2;
      asm_load16(kf[kk], rk, voff);
      asm_load16(vf[kk], rv, voff);
    }
  };

  // ---- epilogue: dK = scale * dK^T^T, dV (key-split partials summed) ----
  auto store_unit = [&](const Unit& x, f32x16* dkacc, f32x16* dvacc, int last_stage) {
    float* comb = reinterpret_cast<float*>(smem + last_stage * Sh::STAGE);
    const int key = x.kt * KT + wv * 32 + l32;
    const int64_t ko = ((int64_t)x.s.k0 * H + x.h) * D;
    TG* dkrow = reinterpret_cast<TG*>(a.dk) + ko + (int64_t)key * HD;
    TG* dvrow = reinterpret_cast<TG*>(a.dv) + ko + (int64_t)key * HD;
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
          store4<TG>(dkrow + col, dkacc[d][i4 * 4] * a.scale, dkacc[d][i4 * 4 + 1] * a.scale,
                     dkacc[d][i4 * 4 + 2] * a.scale, dkacc[d][i4 * 4 + 3] * a.scale);
          store4<TG>(dvrow + col, dvacc[d][i4 * 4], dvacc[d][i4 * 4 + 1], dvacc[d][i4 * 4 + 2],
                     dvacc[d][i4 * 4 + 3]);
        }
    }
  };

  // ---- one step of compute on stage st ----
  auto compute_step = [&](const Unit& x, int t, int st, bf16x8* kf, bf16x8* vf, f32x16* dkacc, f32x16* dvacc,
                          auto&& after_sdp) {
    const char* qt = smem + st * Sh::STAGE;
    const char* ot = qt + Sh::OFF_O;
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
    bf16x8 qa[NKK], oa[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qa[kk] = rows_frag<D, PAD>(qt, wq * 32 + l32, kk, g);
      oa[kk] = rows_frag<D, PAD>(ot, wq * 32 + l32, kk, g);
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      sacc = Elem<bf16>::mma(qa[kk], kf[kk], sacc);
      dpacc = Elem<bf16>::mma(oa[kk], vf[kk], dpacc);
    }
    // keep several fragment reads in flight ahead of the MFMA chain
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int kk = 0; kk < NKK - 3; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    after_sdp();  // K/V fragments are dead from here on in the last step of a unit
    float p[16], ds[16];
    const bool last_step = t + 1 == x.n;
    if constexpr (BIAS) {
      // bias[q][key] for the 16 query rows of this lane (keys past lk carry
      // the next row's values; only their own, unstored columns see them)
      const char* bt = qt + Sh::OFF_B + (wq * 32 + g * 4) * Sh::BT::PITCH + (wv * 32 + l32) * 2;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        p[i] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(bt + acc_row(i, 0) * Sh::BT::PITCH) << 16);
      if (last_step && x.tail) {
        // the tensor's last element may straddle the end of the bias range by
        // half a dword, which the range check drops: reload it
        const rsrc_t rl = make_rsrc(reinterpret_cast<const bf16*>(a.bias) + (a.bias_elems - 1), 2);
        const float last = __uint_as_float((uint32_t)buf_load2(rl, 0) << 16);
        const int key = x.kt * KT + wv * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          p[i] = (key == x.s.lk - 1 && t * QS + wq * 32 + acc_row(i, g) == x.s.lq - 1) ? last : p[i];
      }
    }
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
          p[i] = fast_exp2(fmaf(sacc[i], a.scale_log2, c));
          ds[i] = p[i] * (dpacc[i] - d4[j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float xv = BIAS ? fmaf(sacc[i], a.scale, p[i]) : sacc[i] * a.scale;
        p[i] = act_fwd(ACT, xv);
        ds[i] = act_grad(ACT, xv) * dpacc[i];
      }
    }
    if (last_step) {
      // query rows past the sample end: zero Q, dO and row statistics make
      // their terms vanish unless the bias of another row overflowed P
      const int qrem = x.s.lq - (t * QS + wq * 32);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = acc_row(i, g) < qrem;
        p[i] = ok ? p[i] : 0.0f;
        ds[i] = ok ? ds[i] : 0.0f;
      }
    }
    if constexpr (DBIAS != 0) {
      // dBias[q][key] = dS; rows past the sample end fall outside the
      // descriptor, and a lane whose key is past the end stores out of range
      const int key = x.kt * KT + wv * 32 + l32;
      const rsrc_t rdbr = make_rsrc(reinterpret_cast<const char*>(a.dbias) +
                                        (x.s.bias0 + (int64_t)x.h * x.s.lq * x.s.lk) * ESB,
                                    (uint32_t)x.s.lq * x.s.lk * ESB);
      const uint32_t vb = key < x.s.lk ? (uint32_t)(((t * QS + wq * 32 + g * 4) * x.s.lk + key) * ESB)
                                       : 0x80000000u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t voff = vb + (uint32_t)(((i >> 2) * 8 + (i & 3)) * x.s.lk * ESB);
        if constexpr (DBIAS == 2)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ds[i]), rdbr, voff, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16)ds[i]), rdbr, voff, 0, 0);
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 ph = pack8(&p[s2 * 8]), dh = pack8(&ds[s2 * 8]);
      bf16x8 pl, dl;
      if constexpr (SPLIT) {
        float r1[8], r2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          r1[j] = p[s2 * 8 + j] - (float)ph[j];
          r2[j] = ds[s2 * 8 + j] - (float)dh[j];
        }
        pl = pack8(r1);
        dl = pack8(r2);
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const bf16x8 oa = trans_frag<D, PAD>(ot, wq, s2, d * 32, lane);
        const bf16x8 qa = trans_frag<D, PAD>(qt, wq, s2, d * 32, lane);
        dvacc[d] = Elem<bf16>::mma(oa, ph, dvacc[d]);
        dkacc[d] = Elem<bf16>::mma(qa, dh, dkacc[d]);
        if constexpr (SPLIT) {
          dvacc[d] = Elem<bf16>::mma(oa, pl, dvacc[d]);
          dkacc[d] = Elem<bf16>::mma(qa, dl, dkacc[d]);
        }
      }
    }
  };

  // Wait for the loads of the step about to be computed (and, at a unit
  // boundary, the K/V loads issued in the previous step).  Vector memory
  // operations complete in issue order, so every operation issued after the
  // needed ones may stay in flight: the previous step's prefetch (`recent`)
  // and the dBias stores of the last two steps (S per step, issued after
  // each step's prefetch; the older batch only when no K/V load sits between).
  auto wait_step = [&](bool boundary, int computed, int recent) {
    if constexpr (NS == 3) {
      constexpr int S = DBIAS != 0 ? 16 : 0;
      static_assert(2 * S + L < 64, "vmcnt range");
      const int ns = (computed >= 1 ? 1 : 0) + ((computed >= 2 && !boundary) ? 1 : 0);
      if (recent > 0) {
        if (ns == 2) wait_vmcnt<2 * S + L>();
        else if (ns == 1) wait_vmcnt<S + L>();
        else wait_vmcnt<L>();
      } else {
        if (ns == 2) wait_vmcnt<2 * S>();
        else if (ns == 1) wait_vmcnt<S>();
        else wait_vmcnt<0>();
      }
    } else {
      wait_vmcnt<0>();
    }
  };

  // ---- consumer ----
  if (u_begin >= u_end) return;
  bf16x8 kf[NKK], vf[NKK];
  int cs = 0;        // stage of the next step to compute
  int recent = 0;    // did the previous iteration issue a step (NS == 3)
  int computed = 0;  // steps computed so far
  {
    int u0 = u_begin;
    Unit x0 = fetch(u0);
    while (x0.n == 0 && u0 + 1 < u_end) x0 = fetch(++u0);
    if (x0.n > 0) load_kv(x0, kf, vf);
  }
  for (int j = 0; j < NS - 1; ++j) recent = produce() ? 1 : 0;

  for (int u = u_begin; u < u_end; ++u) {
    const Unit x = fetch(u);
    f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      dkacc[d] = f32x16{};
      dvacc[d] = f32x16{};
    }
    if (x.n > 0) {
      // next unit with steps: its K/V replace this unit's in the last step,
      // right after their last use and before the step's prefetch, so the
      // next iteration's wait (which leaves only that prefetch in flight)
      // covers them
      int un = u + 1;
      Unit xn = x;
      bool has_next = false;
      while (un < u_end) {
        xn = fetch(un);
        if (xn.n > 0) {
          has_next = true;
          break;
        }
        ++un;
      }
      for (int t = 0; t < x.n; ++t) {
        wait_step(t == 0 && computed > 0, computed, recent);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        const bool last = t + 1 == x.n;
        compute_step(x, t, cs, kf, vf, dkacc, dvacc, [&]() {
          if (last && has_next) load_kv(xn, kf, vf);
          recent = produce() ? 1 : 0;
        });
        cs = cs + 1 == NS ? 0 : cs + 1;
        ++computed;
      }
    }
    store_unit(x, dkacc, dvacc, cs == 0 ? NS - 1 : cs - 1);
  }
}

}  // namespace jattn
