#pragma once
// Forward kernel of jagged attention (dense mask), gfx950.
//
// Method: "Training GEM at LLM scale" (Meta engineering post).
//  * section "Jagged Sequence Flash Attention": FlashAttention run directly on
//    jagged tensors; tail rows of Q/K are zero-filled instead of a 2-D -inf
//    mask and the spurious exponentials they add are subtracted afterwards.
//  * section "Generalized Dot-Product Attention (GDPA)": the same kernel with
//    GELU/SiLU applied element-wise in place of softmax, no normalisation.
//
// Work decomposition.  A persistent workgroup (4 waves) walks its slice of a
// host-built unit list; a unit is one (sample, head, q-tile).  Each wave owns
// 32 query rows.  Per K/V tile the workgroup stages K row-major and V
// transposed in LDS (zero rows past the sample end come from buffer loads
// past num_records), then each wave computes
//     S^T = K Q^T          (MFMA 32x32; A = K from LDS, B = Q in registers)
//     online softmax       (each lane holds one query row: stats stay in-lane)
//     O^T += V^T P^T       (A = V^T from LDS, B = P straight from S^T)
// The kv order inside each 32-block of V^T is permuted so that the MFMA
// accumulator layout of S^T is directly the B-operand layout of P.
#include "common.hpp"
#include "kernels.hpp"

namespace jattn {

template <typename TI, int D, int WQ, int WK>
struct FwdShape {
  static constexpr int KP = Elem<TI>::KP;
  static constexpr int KK = 2 * KP;        // contraction length of one MFMA
  static constexpr int NKK = D / KK;       // MFMAs along the head dim
  static constexpr int BM = 32 * WQ;       // query rows per unit
  static constexpr int NBW = (WK == 1) ? 2 : 1;  // 32-key blocks per wave per tile
  static constexpr int BN = 32 * NBW * WK;  // keys per tile
  static constexpr int ND = D / 32;        // 32-wide blocks of the head dim
  static constexpr int CE = 16 / (int)sizeof(TI);  // elements per 16-byte chunk
  static constexpr int CPR = D / CE;       // chunks per row
  static constexpr int CPT = BN * CPR / kThreads;  // chunks per thread per tile
  static constexpr int GRP = CPT < 4 ? CPT : 4;    // rows per transposed write
  static constexpr int KPITCH = D + CE;    // LDS row pitch of K (elements)
  static constexpr int VPITCH = BN + CE;   // LDS row pitch of V^T
  static constexpr int BPITCH = BN + 4;    // LDS row pitch of the bias tile
  static constexpr int BPT = BM * BN / kThreads;  // bias elements per thread
  static_assert(CPT >= 1 && (BN * CPR) % kThreads == 0, "tile/threads mismatch");
  static_assert(kThreads % BN == 0, "bias staging assumes BN | 256");
};

// Value of a probability as the PV MFMA consumes it (bf16 operands are
// rounded to nearest even; fp32 operands are exact).
template <typename TI>
__device__ __forceinline__ float round_p(float x) {
  if constexpr (sizeof(TI) == 2)
    return (float)(bf16)x;
  else
    return x;
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(dst) = v;
}

// Gather element e of GRP consecutive 16-byte chunks (rows) into one packed
// group for the transposed V store.
template <typename TI, int GRP>
struct TGroup;
template <int GRP>
struct TGroup<bf16, GRP> {
  static __device__ __forceinline__ void write(bf16* dst, const i32x4* rows, int e) {
    uint32_t w[GRP];
#pragma unroll
    for (int r = 0; r < GRP; ++r) {
      const uint32_t x = (uint32_t)rows[r][e >> 1];
      w[r] = (e & 1) ? (x >> 16) : (x & 0xffffu);
    }
    if constexpr (GRP == 4) {
      u32x2 v = {w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
      *reinterpret_cast<u32x2*>(dst) = v;
    } else if constexpr (GRP == 2) {
      *reinterpret_cast<uint32_t*>(dst) = w[0] | (w[1] << 16);
    } else {
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w[0];
    }
  }
};
template <int GRP>
struct TGroup<float, GRP> {
  static __device__ __forceinline__ void write(float* dst, const i32x4* rows, int e) {
#pragma unroll
    for (int r = 0; r < GRP; ++r) dst[r] = __int_as_float(rows[r][e]);
  }
};

template <typename TI, typename TO, int D, int WQ, int WK, int ACT, bool BIAS, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdArgs a) {
  using E = Elem<TI>;
  using Sh = FwdShape<TI, D, WQ, WK>;
  constexpr int KP = Sh::KP, KK = Sh::KK, NKK = Sh::NKK, BM = Sh::BM, NBW = Sh::NBW;
  constexpr int BN = Sh::BN, ND = Sh::ND, CE = Sh::CE, CPR = Sh::CPR, CPT = Sh::CPT;
  constexpr int GRP = Sh::GRP, KPITCH = Sh::KPITCH, VPITCH = Sh::VPITCH, BPITCH = Sh::BPITCH;
  constexpr int BPT = Sh::BPT;
  constexpr bool SOFTMAX = (ACT == kSoftmax);
  constexpr int SZ = (int)sizeof(TI);

  constexpr int kStageBytes = SZ * (BN * KPITCH + D * VPITCH + (BIAS ? BM * BPITCH : 0));
  constexpr int kCombineBytes = (WK > 1) ? (int)sizeof(float) * (WK * D * 32 + 3 * WK * 32) : 0;
  constexpr int kSmem = kStageBytes > kCombineBytes ? kStageBytes : kCombineBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  TI* Ks = reinterpret_cast<TI*>(smem);
  TI* Vt = Ks + BN * KPITCH;
  TI* Bs = Vt + D * VPITCH;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wq = wave % WQ, wk = wave / WQ;
  const int l32 = lane & 31, g = lane >> 5;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_end = uniform(a.worker_off[worker + 1]);
  const int HD = a.H * D;

  // staging coordinates: this thread moves chunk column sc of rows sr0..sr0+CPT-1
  const int sc = tid % CPR;
  const int sr0 = (tid / CPR) * CPT;
  // bias staging: column bc, rows br0 + i*(256/BN)
  const int bc = tid % BN;
  const int br0 = tid / BN;

  for (int u = uniform(a.worker_off[worker]); u < u_end; ++u) {
    const i32x4 unit = load_unit(a.units, u);
    const int b = unit[0], h = unit[1], qt = unit[2], ntiles = unit[3];
    const Sample s = load_sample(a.samples, b);
    const int qrow = qt * BM + wq * 32 + l32;  // this lane's query row in the sample

    const TI* qbase = reinterpret_cast<const TI*>(a.q) + ((int64_t)s.q0 * a.H + h) * D;
    const rsrc_t rq = make_rsrc(qbase, (uint32_t)s.lq * HD * SZ);
    typename E::frag qf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint32_t voff = (uint32_t)(qrow * HD + kk * KK + g * KP) * SZ;
      if constexpr (KP == 8) {
        i32x4 x = buf_load16(rq, voff);
        qf[kk] = __builtin_bit_cast(bf16x8, x);
      } else {
        qf[kk] = __uint_as_float(buf_load4(rq, voff));
      }
    }

    const TI* kbase = reinterpret_cast<const TI*>(a.k) + ((int64_t)s.k0 * a.H + h) * D;
    const TI* vbase = reinterpret_cast<const TI*>(a.v) + ((int64_t)s.k0 * a.H + h) * D;
    const rsrc_t rk = make_rsrc(kbase, (uint32_t)s.lk * HD * SZ);
    const rsrc_t rv = make_rsrc(vbase, (uint32_t)s.lk * HD * SZ);
    rsrc_t rb = rk;
    if constexpr (BIAS) {
      const TI* bb = reinterpret_cast<const TI*>(a.bias) + s.bias0 + (int64_t)h * s.lq * s.lk;
      rb = make_rsrc(bb, (uint32_t)s.lq * s.lk * SZ);
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;  // running max (log2 units), softmax only
    bool pad_drop = false;    // the row dropped its padded keys (guard above the epilogue)
    float l_run = 0.0f;       // this lane's partial row sum (exact P, for LSE)
    float lr_run = 0.0f;      // same with P as the PV product sees it (for O)

    // register prefetch of one tile
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
      for (int j = 0; j < CPT; ++j)
        *reinterpret_cast<i32x4*>(&Ks[(sr0 + j) * KPITCH + sc * CE]) = kreg[j];
#pragma unroll
      for (int gq = 0; gq < CPT / GRP; ++gq) {
        const int r = sr0 + gq * GRP;  // first row of the group
        const int pr = (r & ~31) + perm32(r & 31);
#pragma unroll
        for (int e = 0; e < CE; ++e)
          TGroup<TI, GRP>::write(&Vt[(sc * CE + e) * VPITCH + pr], &vreg[gq * GRP], e);
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
      __syncthreads();  // previous tile fully consumed
      stage_to_lds();
      __syncthreads();
      if (t + 1 < ntiles) issue_loads(t + 1);

      // ---- S^T = K Q^T for this wave's key blocks ----
      f32x16 sacc[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int kb = (wk * NBW + nb) * 32;  // key block offset within the tile
        sacc[nb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const TI* src = &Ks[(kb + l32) * KPITCH + kk * KK + g * KP];
          typename E::frag af;
          if constexpr (KP == 8)
            af = *reinterpret_cast<const bf16x8*>(src);
          else
            af = *src;
          sacc[nb] = E::mma(af, qf[kk], sacc[nb]);
        }
      }

      // ---- scores -> P ----
      float p[NBW][16];
      if constexpr (SOFTMAX) {
        float mx = -INFINITY;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = sacc[nb][i] * a.scale_log2;
            if constexpr (BIAS) {
              const int kvl = (wk * NBW + nb) * 32 + acc_row(i, g);
              x += E::to_f32(Bs[(wq * 32 + l32) * BPITCH + kvl]) * kLog2e;
            }
            p[nb][i] = x;
            mx = fmaxf(mx, x);
          }
        }
        if (t + 1 == ntiles) {
          // Guard of the subtraction scheme: keys past the sample end score 0
          // in this last tile; a row whose best valid score is below 0 drops
          // them (p = 0) instead of subtracting their exp terms later, which
          // would cancel (or give NaN once the valid terms underflow).
          const int valid_w = s.lk - (t * BN + wk * NBW * 32);  // valid keys of this wave's blocks
          if (valid_w > 0 && valid_w < NBW * 32) {
            float vm = -INFINITY;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
              for (int i = 0; i < 16; ++i) vm = nb * 32 + acc_row(i, g) < valid_w ? fmaxf(vm, p[nb][i]) : vm;
            vm = wave_xor32_max(vm);
            pad_drop = fmaxf(m_run, vm) < 0.0f;
            if (pad_drop) {
              mx = -INFINITY;
#pragma unroll
              for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                  p[nb][i] = nb * 32 + acc_row(i, g) < valid_w ? p[nb][i] : -INFINITY;
                  mx = fmaxf(mx, p[nb][i]);
                }
            }
          }
        }
        mx = wave_xor32_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        float rs = 0.0f, rsr = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            // O is normalised by the sum of P exactly as the PV product sees
            // it, so that it stays a convex combination of V rows; LSE keeps
            // the exact sum
            const float e = exp2f(p[nb][i] - m_new);
            const float er = round_p<TI>(e);
            p[nb][i] = er;
            rs += e;
            rsr += er;
          }
        }
        l_run = l_run * alpha + rs;
        lr_run = lr_run * alpha + rsr;
        m_run = m_new;
#pragma unroll
        for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
      } else {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = sacc[nb][i] * a.scale;
            if constexpr (BIAS) {
              const int kvl = (wk * NBW + nb) * 32 + acc_row(i, g);
              x += E::to_f32(Bs[(wq * 32 + l32) * BPITCH + kvl]);
            }
            p[nb][i] = act_fwd(ACT, x);
          }
        }
      }

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int kb = (wk * NBW + nb) * 32;
#pragma unroll
        for (int st = 0; st < 16 / KP; ++st) {
          typename E::frag pf, pl;
          if constexpr (KP == 8) {
            pf = pack8(&p[nb][st * 8]);
            if constexpr (SPLIT) {
              float r[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) r[j] = p[nb][st * 8 + j] - (float)pf[j];
              pl = pack8(r);
            }
          } else {
            pf = p[nb][st];
          }
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const TI* src = &Vt[(d * 32 + l32) * VPITCH + kb + g * 16 + st * KP];
            typename E::frag vf;
            if constexpr (KP == 8)
              vf = *reinterpret_cast<const bf16x8*>(src);
            else
              vf = *src;
            oacc[d] = E::mma(vf, pf, oacc[d]);
            if constexpr (SPLIT && KP == 8) oacc[d] = E::mma(vf, pl, oacc[d]);
          }
        }
      }
    }

    // ---- epilogue ----
    float scale_out = 1.0f;
    float lse2 = -INFINITY;
    if constexpr (SOFTMAX) {
      // keys past the sample end read as zero: each adds exp2(0 - m) to l
      int npad = 0;
      if (ntiles > 0 && !pad_drop) {
        const int last0 = (ntiles - 1) * BN;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const int base = last0 + (wk * NBW + nb) * 32;
          const int valid = min(max(s.lk - base, 0), 32);
          npad += 32 - valid;
        }
      }
      // (only with padded keys: without them m may sit far below zero, where
      // 2^-m overflows and 0 * inf would be NaN)
      const float pad_e = npad > 0 ? exp2f(-m_run) : 0.0f;
      l_run = wave_xor32_sum(l_run) - (float)npad * pad_e;
      lr_run = wave_xor32_sum(lr_run) - (float)npad * round_p<TI>(pad_e);
      if (WK > 1 && s.lk <= wk * NBW * 32) {
        // this wave's key blocks lie wholly past the sample end: it holds no
        // term of the row (its zero scores must not set the combined max)
        m_run = -INFINITY;
        l_run = 0.0f;
        lr_run = 0.0f;
      }
      if constexpr (WK == 1) {
        scale_out = (s.lk > 0) ? 1.0f / lr_run : 0.0f;
        lse2 = (s.lk > 0) ? m_run + __log2f(l_run) : -INFINITY;
      }
    }

    TO* obase = reinterpret_cast<TO*>(a.o) + ((int64_t)s.q0 * a.H + h) * D;
    if constexpr (WK == 1) {
      if (qrow < s.lq) {
        TO* orow = obase + (int64_t)qrow * HD;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int col = d * 32 + i4 * 8 + g * 4;
            store4<TO>(orow + col, oacc[d][i4 * 4 + 0] * scale_out, oacc[d][i4 * 4 + 1] * scale_out,
                       oacc[d][i4 * 4 + 2] * scale_out, oacc[d][i4 * 4 + 3] * scale_out);
          }
        }
        if (SOFTMAX && a.lse != nullptr && g == 0)
          a.lse[((int64_t)s.q0 + qrow) * a.H + h] = lse2 * kLn2;
      }
    } else {
      // combine the WK key-split partials of the same 32 query rows in LDS
      static_assert(WQ == 1, "key split assumes one query group");
      float* part = reinterpret_cast<float*>(smem);  // [WK][D][32] partial O
      float* mpart = part + WK * D * 32;             // [WK][32]
      float* lpart = mpart + WK * 32;                // [WK][32]
      float* lrpart = lpart + WK * 32;               // [WK][32]
      __syncthreads();  // all waves done with the last tile
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) part[(wk * D + d * 32 + acc_row(i, g)) * 32 + l32] = oacc[d][i];
      if (g == 0) {
        mpart[wk * 32 + l32] = m_run;
        lpart[wk * 32 + l32] = l_run;
        lrpart[wk * 32 + l32] = lr_run;
      }
      __syncthreads();
      // wave w finishes head-dim columns [w*D/4, (w+1)*D/4) for all 32 rows
      float mall = -INFINITY, lall = 0.0f, lrall = 0.0f;
      float fw[WK];
      if constexpr (SOFTMAX) {
#pragma unroll
        for (int w2 = 0; w2 < WK; ++w2) mall = fmaxf(mall, mpart[w2 * 32 + l32]);
#pragma unroll
        for (int w2 = 0; w2 < WK; ++w2) {
          // a sample without keys has every partial at m = -inf: weight 0
          fw[w2] = (s.lk > 0) ? exp2f(mpart[w2 * 32 + l32] - mall) : 0.0f;
          lall += lpart[w2 * 32 + l32] * fw[w2];
          lrall += lrpart[w2 * 32 + l32] * fw[w2];
        }
      } else {
#pragma unroll
        for (int w2 = 0; w2 < WK; ++w2) fw[w2] = 1.0f;
      }
      const float inv = SOFTMAX ? ((s.lk > 0) ? 1.0f / lrall : 0.0f) : 1.0f;
      constexpr int DC = D / WK;  // columns per wave
      const int row = qt * BM + l32;
      if (row < s.lq) {
        TO* orow = obase + (int64_t)row * HD;
#pragma unroll
        for (int c4 = g * 4; c4 < DC; c4 += 8) {
          float r[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = wave * DC + c4 + j;
            float acc = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < WK; ++w2) acc += part[(w2 * D + col) * 32 + l32] * fw[w2];
            r[j] = acc * inv;
          }
          store4<TO>(orow + wave * DC + c4, r[0], r[1], r[2], r[3]);
        }
        if (SOFTMAX && a.lse != nullptr && wave == 0 && g == 0)
          a.lse[((int64_t)s.q0 + row) * a.H + h] = (s.lk > 0) ? (mall + __log2f(lall)) * kLn2 : -INFINITY;
      }
      __syncthreads();  // combine buffer aliases the next unit's K tile
    }
  }
}

}  // namespace jattn
