// MXFP8 jagged attention backward for gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Method: "Training GEM at LLM scale" (Meta engineering post), section
// "Mixed Ultra-Low-Precision Training", part "Low Precision Flash Attention":
// the backward products are MXFP8 block-scaled too; Q, K, V and dO are
// quantised once in square 32 x 32 blocks, so the products that read them
// transposed (dV = P^T dO, dK = dS^T Q, dQ = dS K) reuse the same scales
// through the transposed codes; the kernels convert P and dS to MXFP8
// themselves ("Jagged Sequence Flash Attention": dQ in its own pass, so
// every gradient element has one writer and no atomics).
//
//   Di     Di = rowsum(dO * O) and LSE * log2(e) per query row (dO from its
//          codes and scales)
//   dK/dV  unit = (sample, head, 128 keys), wave = 32 keys, steps of 64 queries:
//            S = Q K^T, dP = dO V^T       A = Q / dO rows (LDS), B = K / V (registers)
//            P = exp2(S*scale*log2e - LSE*log2e), dS = P (dP - Di)   (or act, act')
//            dV^T += dO^T P, dK^T += Q^T dS   A = dO^T / Q^T (LDS, codes_t), B = P / dS
//          P rounded with the fixed exponent -8 (P <= 1 given the row's LSE;
//          GDPA: per 32 x 32 block), dS with one exponent per 32 x 32 block.
//   dQ     unit = (sample, head, 128 queries), wave = 32 queries, steps of 64 keys:
//            S^T = K Q^T, dP^T = V dO^T   A = K / V rows (LDS), B = Q / dO (registers)
//            dQ^T += K^T dS^T             A = K^T (LDS, codes_t), B = dS
// Keys past the sample end read as zero and get P = dS = 0; query rows past
// it read as zero (Q, dO, row statistics), so their P is finite and their
// dS zero.
#pragma once
#include "mx_impl.hpp"

namespace jattn {

// Eight E4M3 codes (two dwords) to fp32.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// ---------------------------------------------------------------------------
// Di = rowsum(dO * O) per (row, head), dO dequantised from its codes and
// block scales; also LSE * log2(e).  Workgroup = one (32-row block, head);
// D/16 consecutive lanes share a row, 16 features each.
// ---------------------------------------------------------------------------
template <typename TO, int D>
__global__ __launch_bounds__(2 * D) void mx_di_kernel(MxDiArgs a) {
  constexpr int CPR = D / 16;  // lanes per row
  const int r = blockIdx.x / a.H, h = blockIdx.x - r * a.H;
  const int row0 = a.blocks[2 * r], nrows = a.blocks[2 * r + 1];
  const int row = threadIdx.x / CPR, ch = threadIdx.x % CPR;
  const int64_t HD = (int64_t)a.H * D;
  float acc = 0.0f;
  if (row < nrows) {
    const int64_t e0 = (int64_t)(row0 + row) * HD + h * D + ch * 16;
    const u32x4 c = *reinterpret_cast<const u32x4*>(a.dout.codes + e0);
    const int X = (int)a.dout.scales[((int64_t)r * a.H + h) * (D / 32) + ch / 2] - 127;
    const TO* o = reinterpret_cast<const TO*>(a.o) + e0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[4];
      fp8x4_to_f32(c[j], v);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = fmaf(v[k], (float)o[4 * j + k], acc);
    }
    acc = ldexpf(acc, X);
  }
#pragma unroll
  for (int s = CPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < nrows && ch == 0) {
    const int64_t i = (int64_t)(row0 + row) * a.H + h;
    a.di[i] = acc;
    a.lse2[i] = a.lse[i] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the two gradient kernels
// ---------------------------------------------------------------------------
template <int D>
struct MxBwdTiles {
  using RT = PadTile<D / 2, 1>;  // rows of D code bytes, pitch D + 16
  static constexpr int R_BYTES = RT::template bytes<64>();
  static constexpr int TPITCH = 80;  // transposed rows: 64 tokens + 16 pad bytes
  static constexpr int T_NI = (D * 5 + 63) / 64;
  static constexpr int T_BYTES = T_NI * 1024;
};

// HBM -> LDS loader of a transposed 64-token tile [D][64] from codes_t: two
// consecutive 32-token blocks (block b at byte b * BLK of the descriptor).
template <int D>
struct TLoader {
  static constexpr int NI = MxBwdTiles<D>::T_NI;
  static constexpr int NJ = (NI + 3) / 4;
  uint32_t voff[NJ];
  __device__ __forceinline__ void init(int wave, int lane, int64_t BLK) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int s = (wave + 4 * j) * 64 + lane;
      const int d = s / 5, ch = s % 5;
      voff[j] = (ch < 4 && d < D) ? (uint32_t)((ch >> 1) * BLK + d * 32 + (ch & 1) * 16) : 0x80000000u;
    }
  }
  __device__ __forceinline__ void issue(uint32_t tile, const i32x4& r, int wave) const {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int inst = wave + 4 * j;
      if (inst < NI) lds_dma16(r, tile + inst * 1024, voff[j]);
    }
  }
};

// Descriptor of codes_t for head h, token blocks blk0 and blk0 + 1 of a
// sample whose blocks end at blk_last: a block past it reads zero.
template <int D>
__device__ __forceinline__ i32x4 ttile_rsrc(const uint8_t* codes_t, int blk0, int blk_last, int h, int H) {
  const int64_t vb = ((int64_t)blk0 * H + h) * D * 32;
  const int64_t vend = ((int64_t)blk_last * H + h + 1) * D * 32;
  return rsrc_at(rsrc_words(codes_t, 0), vb, vend - vb);
}

// Lane half g's operand of a row operand read from HBM (32x32x64 layout):
// elements 64c + 16g .. +15 and 64c + 32 + 16g .. +15 of the row.
__device__ __forceinline__ i32x8 mx_row_regs(rsrc_t r, uint32_t row_off, int c, int g) {
  const i32x4 lo = buf_load16(r, row_off + c * 64 + g * 16);
  const i32x4 hi = buf_load16(r, row_off + c * 64 + 32 + g * 16);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Largest |x| over a 32x32 accumulator block held by the wave (16 per lane).
__device__ __forceinline__ float block_amax(const float* x) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(x[i]));
  return wave_max64(m);
}

// Round 16 accumulator values (already divided by 2^X) of each of two blocks to
// E4M3 and rearrange them into the operand of lane half g.
__device__ __forceinline__ i32x8 mx_pack_operand(const float (&v)[2][16]) {
  uint32_t w[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) w[b][j] = pack4_fp8(v[b][4 * j], v[b][4 * j + 1], v[b][4 * j + 2], v[b][4 * j + 3]);
  return mx_acc_operand(w);
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <int D, bool SOFTMAX>
struct MxDkdvShape {
  using T = MxBwdTiles<D>;
  static constexpr int OFF_DO = T::R_BYTES;
  static constexpr int OFF_QT = 2 * T::R_BYTES;
  static constexpr int OFF_DOT = OFF_QT + T::T_BYTES;
  static constexpr int OFF_RS = OFF_DOT + T::T_BYTES;  // LSE*log2e [64], Di [64]
  static constexpr int STAGE = OFF_RS + (SOFTMAX ? 512 : 0);
  static constexpr int NS_FIT = 160 * 1024 / STAGE;
  static constexpr int NS = NS_FIT >= 4 ? 4 : NS_FIT;  // ring stages
  static_assert(NS >= 2, "two stages at least");
  static constexpr int SMEM = NS * STAGE;
};

// Unit record of the MXFP8 kernels: head, tile, steps, sample fields and the
// sample's first row blocks of Q and K (entries 6 and 7 of its table entry),
// read with scalar loads.
struct MxUnit {
  int h, tile, n;
  Sample s;
  int qblk0, kblk0;
};
__device__ __forceinline__ MxUnit mx_fetch(const int32_t* units, const int32_t* samples, int u) {
  MxUnit x;
  const i32x4 un = sload4(units, u);
  x.h = un[1];
  x.tile = un[2];
  x.n = un[3];
  x.s = sload_sample(samples, un[0]);
  const i32x4 y = sload4(samples, 2 * un[0] + 1);
  x.qblk0 = y[2];
  x.kblk0 = y[3];
  return x;
}

// Both gradient kernels: the tiles of a step travel HBM -> LDS into a ring of
// NS stages filled by a producer cursor that runs NS - 1 steps ahead across
// unit boundaries (descriptors set up once per unit, advanced per step; each
// step waits only for its own loads, with per-wave counts); the register
// operands of the next unit with steps are loaded in the last step of a unit
// (its own instance, so the loop over the other steps carries no register
// loads for the compiler to wait on); gradients are stored with buffer
// stores from every lane, so the counts do not depend on the data.
template <typename TG, int D, int ACT>
__global__ __launch_bounds__(256, 1) void mx_dkdv_kernel(MxBwdArgs a) {
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  using Sh = MxDkdvShape<D, SOFTMAX>;
  using Tl = MxBwdTiles<D>;
  constexpr int NC = D / 64, ND = D / 32, KT = 128, QS = 64, NS = Sh::NS;
  __shared__ __attribute__((aligned(1024))) char smem[Sh::SMEM];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_begin = sload1(a.worker_off, worker);
  const int u_end = sload1(a.worker_off, worker + 1);
  const int H = a.H, HD = H * D;
  const int64_t BLK = (int64_t)H * D * 32;
  const uint32_t smem_lds = lds_addr(smem);
  RowLoader<D / 2, 1, QS, 4> rload;
  rload.init(wave, lane, HD / 2);
  TLoader<D> tload;
  tload.init(wave, lane, BLK);
  if (u_begin >= u_end) return;
  auto fetch = [&](int u) { return mx_fetch(a.units, a.samples, u); };

  // ---- producer: Q, dO rows, their transposed tiles and the row statistics
  // of query rows 64t .. of the unit's (sample, head) ----
  constexpr int RNI = decltype(rload)::NI, TNI = Tl::T_NI;
  const int step_ops = 2 * loads_of(RNI, wave, 4) + 2 * loads_of(TNI, wave, 4) + (SOFTMAX && wave < 2 ? 1 : 0);
  constexpr int MIN_OPS = 2 * loads_of(RNI, 3, 4) + 2 * loads_of(TNI, 3, 4);  // wave 3: no row statistics
  constexpr int LOOK = NS - 1;
  constexpr int WAIT_N = (LOOK - 1) * MIN_OPS < 63 ? (LOOK - 1) * MIN_OPS : 63;
  VmLedger<LOOK, WAIT_N> ring;
  int pu = u_begin, pt = 0, pn = 0, pst = 0;
  Walker<false> w_q, w_do, w_qt, w_dot, w_rs;
  auto start_unit = [&](const MxUnit& x) {
    const int64_t qo = ((int64_t)x.s.q0 * H + x.h) * D;
    w_q.start(a.q.codes, qo, (int64_t)x.s.lq * HD);
    w_do.start(a.dout.codes, qo, (int64_t)x.s.lq * HD);
    // token blocks qblk0 + 2t, + 2t + 1; the descriptor ends with the sample's
    // last block, so a block past it reads zero
    const int nqb = (x.s.lq + 31) >> 5;
    const int64_t vb = ((int64_t)x.qblk0 * H + x.h) * D * 32;
    const int64_t vend = ((int64_t)(x.qblk0 + nqb - 1) * H + x.h + 1) * D * 32;
    w_qt.start(a.q.codes_t, vb, vend - vb);
    w_dot.start(a.dout.codes_t, vb, vend - vb);
    // LSE * log2e (wave 0) or Di (wave 1); rows past the sample end read zero
    if constexpr (SOFTMAX)
      w_rs.start(wave == 0 ? a.lse2 : a.di, ((int64_t)x.s.q0 * H + x.h) * 4, (int64_t)x.s.lq * H * 4);
  };
  MxUnit pinfo = fetch(u_begin);
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
      rload.issue(sb, w_q.words(), wave);
      rload.issue(sb + Sh::OFF_DO, w_do.words(), wave);
      tload.issue(sb + Sh::OFF_QT, w_qt.words(), wave);
      tload.issue(sb + Sh::OFF_DOT, w_dot.words(), wave);
      if constexpr (SOFTMAX) {
        if (wave < 2) lds_dma4(w_rs.words(), sb + Sh::OFF_RS + wave * 256, (uint32_t)lane * H * 4);
      }
      w_q.advance((int64_t)QS * HD);
      w_do.advance((int64_t)QS * HD);
      w_qt.advance(2 * BLK);
      w_dot.advance(2 * BLK);
      if constexpr (SOFTMAX) w_rs.advance((int64_t)QS * H * 4);
      ++pt;
      pst = pst + 1 == NS ? 0 : pst + 1;
      ring.produced(step_ops);
    } else {
      ring.produced(0);
    }
  };

  // K and V rows of this wave's keys (B operands) and their scale bytes
  i32x8 kf[NC], vf[NC];
  int ksc[NC], vsc[NC];
  auto load_kv = [&](const MxUnit& x) {
    const int key = x.tile * KT + wave * 32 + l32;
    const int64_t base = ((int64_t)x.s.k0 * H + x.h) * D;
    const rsrc_t rk = make_rsrc(a.k.codes + base, (uint32_t)x.s.lk * HD);
    const rsrc_t rv = make_rsrc(a.v.codes + base, (uint32_t)x.s.lk * HD);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = mx_row_regs(rk, (uint32_t)key * HD, c, g);
      vf[c] = mx_row_regs(rv, (uint32_t)key * HD, c, g);
    }
    const int nkb = (x.s.lk + 31) >> 5;
    const int kbk = x.kblk0 + min(x.tile * 4 + wave, nkb - 1);
    const uint32_t kw = mx_scale_word<D>(a.k.scales, kbk, x.h, H);
    const uint32_t vw = mx_scale_word<D>(a.v.scales, kbk, x.h, H);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ksc[c] = scale_byte(kw, 2 * c + g);
      vsc[c] = scale_byte(vw, 2 * c + g);
    }
  };
  auto load_next_kv = [&](int from) {
    for (int un = from; un < u_end; ++un) {
      const MxUnit xn = fetch(un);
      if (xn.n > 0) {
        load_kv(xn);
        break;
      }
    }
  };
  // the first unit's K/V have landed before anything else is issued
  load_next_kv(u_begin);
  wait_vmcnt<0>();
  for (int j = 0; j < LOOK; ++j) produce();
  int stage = 0;

  for (int u = u_begin; u < u_end; ++u) {
    const MxUnit x = fetch(u);
    const int n = x.n;
    const int nqb = (x.s.lq + 31) >> 5;
    const int key = x.tile * KT + wave * 32 + l32;  // this lane's key (column of S)
    const bool key_ok = key < x.s.lk;

    f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      dkacc[d] = f32x16{};
      dvacc[d] = f32x16{};
    }
    auto step = [&](auto last_tag, int t) {
      constexpr bool LAST = decltype(last_tag)::value;
      ring.wait_oldest();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // step t is in LDS; every wave is done with the stage produce() refills
      __builtin_amdgcn_sched_barrier(0);
      produce();
      const char* sb = smem + stage * Sh::STAGE;
      int qw[2], dw[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int blk = x.qblk0 + min(2 * t + qb, nqb - 1);
        qw[qb] = (int)mx_scale_word<D>(a.q.scales, blk, x.h, H);
        dw[qb] = (int)mx_scale_word<D>(a.dout.scales, blk, x.h, H);
      }
      // ---- S = Q K^T and dP = dO V^T; lane (key, g) holds queries qb*32 + acc_row(i, g) ----
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        sacc[qb] = f32x16{};
        pacc[qb] = f32x16{};
        const char* qrow = sb + Tl::RT::off(qb * 32 + l32, 0);
        const char* drow = sb + Sh::OFF_DO + Tl::RT::off(qb * 32 + l32, 0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sacc[qb] = mx_mma(mx_frag(qrow + c * 64, g), kf[c], sacc[qb], scale_byte(qw[qb], 2 * c + g), ksc[c]);
          pacc[qb] = mx_mma(mx_frag(drow + c * 64, g), vf[c], pacc[qb], scale_byte(dw[qb], 2 * c + g), vsc[c]);
        }
      }
      // K and V are free after the unit's last S/dP: the next unit with steps loads its own
      if constexpr (LAST) load_next_kv(u + 1);
      // ---- P, dS ----
      float p[2][16], ds[2][16];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float lse2[16], di[16];
        if constexpr (SOFTMAX) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int q = qb * 32 + 8 * j + 4 * g;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(sb + Sh::OFF_RS + q * 4);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(sb + Sh::OFF_RS + 256 + q * 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              lse2[4 * j + k] = l4[k];
              di[4 * j + k] = d4[k];
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (SOFTMAX) {
            p[qb][i] = fast_exp2(fmaf(sacc[qb][i], a.scale_log2, -lse2[i]));
            ds[qb][i] = p[qb][i] * (pacc[qb][i] - di[i]);
          } else {
            const float xv = sacc[qb][i] * a.scale;
            p[qb][i] = act_fwd(ACT, xv);
            ds[qb][i] = act_grad(ACT, xv) * pacc[qb][i];
          }
          p[qb][i] = key_ok ? p[qb][i] : 0.0f;
          ds[qb][i] = key_ok ? ds[qb][i] : 0.0f;
        }
      }
      // ---- P and dS to E4M3: one exponent per 32 x 32 block (P of softmax: -8) ----
      int xp[2], xs[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        xp[qb] = SOFTMAX ? -8 : mx_scale_exp(block_amax(p[qb]));
        xs[qb] = mx_scale_exp(block_amax(ds[qb]));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[qb][i] = ldexpf(p[qb][i], -xp[qb]);
          ds[qb][i] = ldexpf(ds[qb][i], -xs[qb]);
        }
      }
      const i32x8 pop = mx_pack_operand(p), sop = mx_pack_operand(ds);
      const int psc = (g ? xp[1] : xp[0]) + 127, ssc = (g ? xs[1] : xs[0]) + 127;
      // ---- dV^T += dO^T P, dK^T += Q^T dS ----
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const int aq = scale_byte(g ? qw[1] : qw[0], d), ad = scale_byte(g ? dw[1] : dw[0], d);
        dvacc[d] = mx_mma(mx_frag(sb + Sh::OFF_DOT + (d * 32 + l32) * Tl::TPITCH, g), pop, dvacc[d], ad, psc);
        dkacc[d] = mx_mma(mx_frag(sb + Sh::OFF_QT + (d * 32 + l32) * Tl::TPITCH, g), sop, dkacc[d], aq, ssc);
      }
      stage = stage + 1 == NS ? 0 : stage + 1;
    };
    if (n > 0) {
      for (int t = 0; t + 1 < n; ++t) step(std::false_type{}, t);
      step(std::true_type{}, n - 1);
    }
    // ---- store dK = scale * dK^T^T, dV: lane (key, g) holds features d*32 + acc_row(i, g) ----
    {
      const int64_t base = ((int64_t)x.s.k0 * H + x.h) * D;
      const uint32_t bytes = (uint32_t)x.s.lk * HD * (uint32_t)sizeof(TG);
      const rsrc_t rdk = make_rsrc(reinterpret_cast<const TG*>(a.dk) + base, bytes);
      const rsrc_t rdv = make_rsrc(reinterpret_cast<const TG*>(a.dv) + base, bytes);
      const uint32_t vrow = key_ok ? (uint32_t)(key * HD) * (uint32_t)sizeof(TG) : 0x80000000u;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const uint32_t off = vrow + (uint32_t)(d * 32 + i4 * 8 + g * 4) * (uint32_t)sizeof(TG);
          buf_store4<TG>(rdk, off, a.scale * dkacc[d][i4 * 4], a.scale * dkacc[d][i4 * 4 + 1],
                         a.scale * dkacc[d][i4 * 4 + 2], a.scale * dkacc[d][i4 * 4 + 3]);
          buf_store4<TG>(rdv, off, dvacc[d][i4 * 4], dvacc[d][i4 * 4 + 1], dvacc[d][i4 * 4 + 2], dvacc[d][i4 * 4 + 3]);
        }
      ring.counted(2 * ND * 4);
    }
  }
  // every production was acquired; only stores can still be in flight
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
struct MxDqShape {
  using T = MxBwdTiles<D>;
  static constexpr int OFF_V = T::R_BYTES;
  static constexpr int OFF_KT = 2 * T::R_BYTES;
  static constexpr int STAGE = OFF_KT + T::T_BYTES;
  static constexpr int NS_FIT = 160 * 1024 / STAGE;
  static constexpr int NS = NS_FIT >= 4 ? 4 : NS_FIT;  // ring stages
  static_assert(NS >= 2, "two stages at least");
  static constexpr int SMEM = NS * STAGE;
};

template <typename TG, int D, int ACT>
__global__ __launch_bounds__(256, 1) void mx_dq_kernel(MxBwdArgs a) {
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  using Sh = MxDqShape<D>;
  using Tl = MxBwdTiles<D>;
  constexpr int NC = D / 64, ND = D / 32, BM = 128, BN = 64, NS = Sh::NS;
  __shared__ __attribute__((aligned(1024))) char smem[Sh::SMEM];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_begin = sload1(a.worker_off, worker);
  const int u_end = sload1(a.worker_off, worker + 1);
  const int H = a.H, HD = H * D;
  const int64_t BLK = (int64_t)H * D * 32;
  const uint32_t smem_lds = lds_addr(smem);
  RowLoader<D / 2, 1, BN, 4> rload;
  rload.init(wave, lane, HD / 2);
  TLoader<D> tload;
  tload.init(wave, lane, BLK);
  if (u_begin >= u_end) return;
  auto fetch = [&](int u) { return mx_fetch(a.units, a.samples, u); };

  // ---- producer: K, V rows and the transposed K tile of keys 64t .. ----
  constexpr int RNI = decltype(rload)::NI, TNI = Tl::T_NI;
  const int step_ops = 2 * loads_of(RNI, wave, 4) + loads_of(TNI, wave, 4);
  constexpr int MIN_OPS = 2 * loads_of(RNI, 3, 4) + loads_of(TNI, 3, 4);
  constexpr int LOOK = NS - 1;
  constexpr int WAIT_N = (LOOK - 1) * MIN_OPS < 63 ? (LOOK - 1) * MIN_OPS : 63;
  VmLedger<LOOK, WAIT_N> ring;
  int pu = u_begin, pt = 0, pn = 0, pst = 0;
  Walker<false> w_k, w_v, w_kt;
  auto start_unit = [&](const MxUnit& x) {
    const int64_t ko = ((int64_t)x.s.k0 * H + x.h) * D;
    w_k.start(a.k.codes, ko, (int64_t)x.s.lk * HD);
    w_v.start(a.v.codes, ko, (int64_t)x.s.lk * HD);
    const int nkb = (x.s.lk + 31) >> 5;
    const int64_t vb = ((int64_t)x.kblk0 * H + x.h) * D * 32;
    const int64_t vend = ((int64_t)(x.kblk0 + nkb - 1) * H + x.h + 1) * D * 32;
    w_kt.start(a.k.codes_t, vb, vend - vb);
  };
  MxUnit pinfo = fetch(u_begin);
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
      rload.issue(sb, w_k.words(), wave);
      rload.issue(sb + Sh::OFF_V, w_v.words(), wave);
      tload.issue(sb + Sh::OFF_KT, w_kt.words(), wave);
      w_k.advance((int64_t)BN * HD);
      w_v.advance((int64_t)BN * HD);
      w_kt.advance(2 * BLK);
      ++pt;
      pst = pst + 1 == NS ? 0 : pst + 1;
      ring.produced(step_ops);
    } else {
      ring.produced(0);
    }
  };

  // Q and dO rows of this lane's query (B operands), scale bytes, row statistics
  i32x8 qf[NC], df[NC];
  int qsc[NC], dsc[NC];
  float lse2 = 0.0f, di = 0.0f;
  auto load_rows = [&](const MxUnit& x) {
    const int q = x.tile * BM + wave * 32 + l32;
    const int64_t base = ((int64_t)x.s.q0 * H + x.h) * D;
    const rsrc_t rq = make_rsrc(a.q.codes + base, (uint32_t)x.s.lq * HD);
    const rsrc_t rd = make_rsrc(a.dout.codes + base, (uint32_t)x.s.lq * HD);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = mx_row_regs(rq, (uint32_t)q * HD, c, g);
      df[c] = mx_row_regs(rd, (uint32_t)q * HD, c, g);
    }
    const int nqb = (x.s.lq + 31) >> 5;
    const int qbk = x.qblk0 + min(x.tile * 4 + wave, nqb - 1);
    const uint32_t qw = mx_scale_word<D>(a.q.scales, qbk, x.h, H);
    const uint32_t dw = mx_scale_word<D>(a.dout.scales, qbk, x.h, H);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qsc[c] = scale_byte(qw, 2 * c + g);
      dsc[c] = scale_byte(dw, 2 * c + g);
    }
    if constexpr (SOFTMAX) {
      // rows past the sample end read as zero
      const uint32_t rec = (uint32_t)x.s.lq * H * 4;
      lse2 = __uint_as_float(buf_load4(make_rsrc(a.lse2 + (int64_t)x.s.q0 * H + x.h, rec), (uint32_t)q * H * 4));
      di = __uint_as_float(buf_load4(make_rsrc(a.di + (int64_t)x.s.q0 * H + x.h, rec), (uint32_t)q * H * 4));
    }
  };
  auto load_next_rows = [&](int from) {
    for (int un = from; un < u_end; ++un) {
      const MxUnit xn = fetch(un);
      if (xn.n > 0) {
        load_rows(xn);
        break;
      }
    }
  };
  // the first unit's rows have landed before anything else is issued
  load_next_rows(u_begin);
  wait_vmcnt<0>();
  for (int j = 0; j < LOOK; ++j) produce();
  int stage = 0;

  for (int u = u_begin; u < u_end; ++u) {
    const MxUnit x = fetch(u);
    const int n = x.n;
    const int nkb = (x.s.lk + 31) >> 5;
    const int q = x.tile * BM + wave * 32 + l32;  // this lane's query row
    // this unit's row statistics (the next unit's may load during its last step)
    const float lse2_u = lse2, di_u = di;

    f32x16 dqacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) dqacc[d] = f32x16{};
    auto step = [&](auto last_tag, int t) {
      constexpr bool LAST = decltype(last_tag)::value;
      ring.wait_oldest();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();  // step t is in LDS; every wave is done with the stage produce() refills
      __builtin_amdgcn_sched_barrier(0);
      produce();
      const char* sb = smem + stage * Sh::STAGE;
      int kw[2], vw[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int blk = x.kblk0 + min(2 * t + kb, nkb - 1);
        kw[kb] = (int)mx_scale_word<D>(a.k.scales, blk, x.h, H);
        vw[kb] = (int)mx_scale_word<D>(a.v.scales, blk, x.h, H);
      }
      // ---- S^T = K Q^T, dP^T = V dO^T; lane (query, g) holds keys kb*32 + acc_row(i, g) ----
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        pacc[kb] = f32x16{};
        const char* krow = sb + Tl::RT::off(kb * 32 + l32, 0);
        const char* vrow = sb + Sh::OFF_V + Tl::RT::off(kb * 32 + l32, 0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sacc[kb] = mx_mma(mx_frag(krow + c * 64, g), qf[c], sacc[kb], scale_byte(kw[kb], 2 * c + g), qsc[c]);
          pacc[kb] = mx_mma(mx_frag(vrow + c * 64, g), df[c], pacc[kb], scale_byte(vw[kb], 2 * c + g), dsc[c]);
        }
      }
      // Q and dO are free after the unit's last S^T / dP^T: the next unit with steps loads its own
      if constexpr (LAST) load_next_rows(u + 1);
      float ds[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kbase = t * BN + kb * 32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float v;
          if constexpr (SOFTMAX) {
            v = fast_exp2(fmaf(sacc[kb][i], a.scale_log2, -lse2_u)) * (pacc[kb][i] - di_u);
          } else {
            v = act_grad(ACT, sacc[kb][i] * a.scale) * pacc[kb][i];
          }
          ds[kb][i] = kbase + acc_row(i, g) < x.s.lk ? v : 0.0f;  // keys past the end: none
        }
      }
      // ---- dS to E4M3, one exponent per 32 x 32 block; dQ^T += K^T dS^T ----
      int xs[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        xs[kb] = mx_scale_exp(block_amax(ds[kb]));
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[kb][i] = ldexpf(ds[kb][i], -xs[kb]);
      }
      const i32x8 sop = mx_pack_operand(ds);
      const int ssc = (g ? xs[1] : xs[0]) + 127;
#pragma unroll
      for (int d = 0; d < ND; ++d)
        dqacc[d] = mx_mma(mx_frag(sb + Sh::OFF_KT + (d * 32 + l32) * Tl::TPITCH, g), sop, dqacc[d],
                          scale_byte(g ? kw[1] : kw[0], d), ssc);
      stage = stage + 1 == NS ? 0 : stage + 1;
    };
    if (n > 0) {
      for (int t = 0; t + 1 < n; ++t) step(std::false_type{}, t);
      step(std::true_type{}, n - 1);
    }
    {
      const rsrc_t rq = make_rsrc(reinterpret_cast<const TG*>(a.dq) + ((int64_t)x.s.q0 * H + x.h) * D,
                                  (uint32_t)x.s.lq * HD * (uint32_t)sizeof(TG));
      const uint32_t vrow = q < x.s.lq ? (uint32_t)(q * HD) * (uint32_t)sizeof(TG) : 0x80000000u;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          buf_store4<TG>(rq, vrow + (uint32_t)(d * 32 + i4 * 8 + g * 4) * (uint32_t)sizeof(TG),
                         a.scale * dqacc[d][i4 * 4], a.scale * dqacc[d][i4 * 4 + 1], a.scale * dqacc[d][i4 * 4 + 2],
                         a.scale * dqacc[d][i4 * 4 + 3]);
      ring.counted(ND * 4);
    }
  }
  // every production was acquired; only stores can still be in flight
  wait_vmcnt<0>();
}

}  // namespace jattn
