// BlockAttention kernels (fixed 64-token block-diagonal mask), gfx950.
//
// Method: "Training GEM at LLM scale" (Meta engineering post), section
// "BlockAttention": each 64-token query block attends only to the key/value
// block with the same index, so attention splits into independent 64 x 64
// problems.  A dedicated kernel then needs no online-softmax correction, no
// logsumexp written to memory and no separate Di pass.
//
// Forward : one wave per block.  K and V of the block go straight from HBM
//           into the wave's LDS (buffer loads with LDS destination; rows past
//           the sample end come back as zero), Q goes to registers.  The full
//           64-key softmax row lives in one lane, so one pass computes m, l
//           and P; the zero rows of a partial last block are removed by
//           subtracting their exp(0 - m) terms.
// Backward: two waves per block, one block per workgroup (two workgroups
//           share a CU and run independently).  Phase 1, lane =
//           query row: S^T, softmax, dP^T, Di = sum_j P dP (in-tile), dS,
//           dQ = dS K.  Phase 2, lane = key row: S, dP again, P from the
//           phase-1 row statistics, dV = P^T dO, dK = dS^T Q.
// Operands that are contracted along rows (V^T, K^T, Q^T, dO^T) are read
// from the row-major LDS tiles with ds_read_b64_tr_b16.
//
// Rotary position embedding (ROPE; same section: the RoPE backward is fused
// into the block-attention epilogue and the gradients stay in fp32
// registers).  Rotate-half pairs (j, j + D/2) at position m (token index in
// the sample) turn by m * theta_j, theta_j = base^(-2j/D) (fp64 table in the
// plan).  The forward rotates Q in registers and K in LDS after they land;
// the backward rotates the Q and K tiles in LDS once, and applies the
// transposed rotation to dQ and dK in the accumulator registers before the
// store.  The angle is reduced to [-pi, pi] in fp64, then sine and cosine
// are taken in fp32.
#pragma once
#include "common.hpp"
#include "fwd_impl.hpp"
#include "kernels.hpp"

namespace jattn {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// Row-major bf16 tile in LDS with 16-byte chunks XOR-swizzled per row.
template <int D>
struct Tile {
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int RB = D * 2;         // bytes per row
  static constexpr int BYTES = 64 * RB;    // 64 rows
  static __device__ __forceinline__ int swz(int r) { return r & (CPR - 1); }
  // byte offset of element (r, col) (col multiple of 4)
  static __device__ __forceinline__ int off(int r, int col) {
    const int c = col >> 3;
    return r * RB + ((c ^ swz(r)) << 4) + ((col & 4) << 1);
  }
};

// Issue the loads of one 64-row tile (rows row0.. of a sample/head) straight
// into LDS.  `part`/`nparts` split the CPR instructions among waves.
template <int D>
__device__ __forceinline__ void load_tile_async(char* lds_tile, rsrc_t r, int row0, int HD, int lane, int part,
                                                int nparts) {
  using T = Tile<D>;
  constexpr int RPI = 64 / T::CPR;  // rows per instruction (64 lanes x 16 B)
  for (int inst = part; inst < T::CPR; inst += nparts) {
    const int rr = inst * RPI + lane / T::CPR;  // tile row this lane fills
    const int p = lane % T::CPR;                // LDS chunk position in that row
    const int c = p ^ T::swz(rr);               // logical chunk that belongs there
    const uint32_t voff = (uint32_t)((row0 + rr) * HD + c * 8) * 2;
#if __HIP_DEVICE_COMPILE__
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_tile + inst * 1024), 16,
                                             voff, 0, 0, 0);
#endif
  }
}

__device__ __forceinline__ void wait_vmem() {
  // s_waitcnt vmcnt(0): buffer loads into LDS have landed
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ void wait_lds() {
  // s_waitcnt lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_s_waitcnt(0xC07F);
}

// theta_j from the workgroup's LDS copy of the plan's table
__device__ __forceinline__ double rope_theta(const double* t, int j) { return t[j]; }

// copy the D/2 angles of the plan's table into LDS (before a barrier)
template <int D>
__device__ __forceinline__ void stage_theta(double* dst, const double* src) {
  for (int j = threadIdx.x; j < D / 2; j += blockDim.x) dst[j] = src[j];
}

// cos and sin of m * theta: the angle is formed and reduced to [-pi, pi] in
// fp64 (positions reach 2^25, where an fp32 angle would be off by radians)
__device__ __forceinline__ void rope_cs(int m, double theta, float& c, float& s) {
  constexpr double kTwoPi = 6.283185307179586;
  const double a = (double)m * theta;
  const float r = (float)fma(-rint(a * (1.0 / kTwoPi)), kTwoPi, a);
  __sincosf(r, &s, &c);
}

// Rotate one row of a 64-row LDS tile in place (this lane's row `row`, at
// position m): chunk pairs (cc, cc + CPR/2).
template <int D>
__device__ __forceinline__ void rope_rows_lds(char* tile, const double* theta, int row, int m) {
  using T = Tile<D>;
#pragma unroll 2
  for (int cc = 0; cc < T::CPR / 2; ++cc) {
    bf16x8* p1 = reinterpret_cast<bf16x8*>(tile + T::off(row, cc * 8));
    bf16x8* p2 = reinterpret_cast<bf16x8*>(tile + T::off(row, cc * 8 + D / 2));
    bf16x8 x1 = *p1, x2 = *p2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c, s;
      rope_cs(m, rope_theta(theta, cc * 8 + e), c, s);
      const float a1 = (float)x1[e], a2 = (float)x2[e];
      x1[e] = (bf16)(a1 * c - a2 * s);
      x2[e] = (bf16)(a2 * c + a1 * s);
    }
    *p1 = x1;
    *p2 = x2;
  }
}

// Backward angles of one lane: the lane's row (query in phase 1, key in
// phase 2: the same position m) and the pair columns
//     j(n) = (n / 4) * 8 + 4 g + n % 4,   n < D/4,
// which are exactly the first-half columns of the lane's accumulator slots
// (slot i of block d is column d*32 + acc_row(i, g), i.e. n = d*16 + i).
template <int D>
__device__ __forceinline__ void rope_lane_angles(const double* theta, int m, int g, float* rc, float* rs) {
#pragma unroll
  for (int n = 0; n < D / 4; ++n) rope_cs(m, rope_theta(theta, (n >> 2) * 8 + g * 4 + (n & 3)), rc[n], rs[n]);
}

// Rotate the lane's columns j(n) (and j(n) + D/2) of row `row` of an LDS tile.
template <int D>
__device__ __forceinline__ void rope_lane_lds(char* tile, int row, int g, const float* rc, const float* rs) {
  using T = Tile<D>;
#pragma unroll
  for (int q = 0; q < D / 16; ++q) {
    bf16x4* p1 = reinterpret_cast<bf16x4*>(tile + T::off(row, q * 8 + g * 4));
    bf16x4* p2 = reinterpret_cast<bf16x4*>(tile + T::off(row, q * 8 + g * 4 + D / 2));
    bf16x4 x1 = *p1, x2 = *p2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = rc[q * 4 + e], s = rs[q * 4 + e];
      const float a1 = (float)x1[e], a2 = (float)x2[e];
      x1[e] = (bf16)(a1 * c - a2 * s);
      x2[e] = (bf16)(a2 * c + a1 * s);
    }
    *p1 = x1;
    *p2 = x2;
  }
}

// Transposed rotation of a gradient row held in accumulator order: slot i of
// block d (n = d*16 + i) pairs with block d + ND/2; with one block (D = 32)
// the pairs are slots i and i + 8 (columns c, c + 16).
template <int ND>
__device__ __forceinline__ void rope_back_acc(f32x16* acc, const float* rc, const float* rs) {
  constexpr int NB = ND > 1 ? ND / 2 : 1;   // blocks holding first halves
  constexpr int NI = ND > 1 ? 16 : 8;       // their slots holding first halves
  constexpr int D2 = ND > 1 ? ND / 2 : 0, I2 = ND > 1 ? 0 : 8;  // partner: block d + D2, slot i + I2
#pragma unroll
  for (int d = 0; d < NB; ++d)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float c = rc[d * 16 + i], s = rs[d * 16 + i];
      const float a1 = acc[d][i], a2 = acc[d + D2][i + I2];
      acc[d][i] = a1 * c + a2 * s;
      acc[d + D2][i + I2] = a2 * c - a1 * s;
    }
}

// bf16 fragment from 8 consecutive accumulator slots
__device__ __forceinline__ bf16x8 pack8_from(const f32x16& v, int off) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)v[off + j];
  return r;
}

// A/B fragment of a row operand: lane (row = base + l%32, k chunk kk*2 + g).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int row, int kk, int g) {
  return *reinterpret_cast<const bf16x8*>(tile + Tile<D>::off(row, kk * 16 + g * 8));
}

// A fragment of a transposed operand X^T (32 columns of X x 16 rows of X):
// lane l gets X[rows][col0 + l%32] for the 8 rows that the accumulator slot
// order of block `blk`, step `st` assigns to lane half g.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int blk, int st, int col0, int lane) {
  const int i = lane & 15, grp = (lane >> 4) & 1, g = lane >> 5;
  const int col = col0 + 16 * grp + 4 * (i & 3);
  const int r1 = blk * 32 + 16 * st + 4 * g + (i >> 2);
  v4i16 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
#if __HIP_DEVICE_COMPILE__
  lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + Tile<D>::off(r1, col)));
  hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + Tile<D>::off(r1 + 8, col)));
#endif
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// forward: one wave = one 64 x 64 block
// ---------------------------------------------------------------------------
template <typename TO, int D, bool ROPE = false>
__global__ __launch_bounds__(kThreads, 1) void block_fwd_kernel(FwdArgs a) {
  using T = Tile<D>;
  constexpr int NKK = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[4 * 2 * T::BYTES];
  __shared__ double theta_s[ROPE ? D / 2 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  if constexpr (ROPE) {
    stage_theta<D>(theta_s, a.rope_theta);
    __syncthreads();
  }
  char* kt = smem + wave * 2 * T::BYTES;
  char* vt = kt + T::BYTES;
  // two waves share one worker (wave pair) and take alternate units of it
  const int worker = xcd_worker(blockIdx.x, gridDim.x) * 2 + (wave >> 1);
  const int u_end = uniform(a.worker_off[worker + 1]);
  const int HD = a.H * D;

  for (int u = a.worker_off[worker] + (wave & 1); u < u_end; u += 2) {
    const i32x4 unit = load_unit(a.units, u);
    const int b = unit[0], h = unit[1], t = unit[2];
    const Sample s = load_sample(a.samples, b);
    const int row0 = t * 64;
    const int r = min(64, s.lq - row0);  // valid rows of this block
    const int64_t base = ((int64_t)(s.k0 + row0) * a.H + h) * D;
    const rsrc_t rk = make_rsrc(reinterpret_cast<const bf16*>(a.k) + base, (uint32_t)r * HD * 2);
    const rsrc_t rv = make_rsrc(reinterpret_cast<const bf16*>(a.v) + base, (uint32_t)r * HD * 2);
    const int64_t qbase = ((int64_t)(s.q0 + row0) * a.H + h) * D;
    const rsrc_t rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + qbase, (uint32_t)r * HD * 2);

    __builtin_amdgcn_wave_barrier();
    load_tile_async<D>(kt, rk, 0, HD, lane, 0, 1);
    load_tile_async<D>(vt, rv, 0, HD, lane, 0, 1);
    bf16x8 qf[2][NKK];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        qf[qb][kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)((qb * 32 + l32) * HD + kk * 16 + g * 8) * 2));
    if constexpr (ROPE) {
      // Q in registers: element e of fragment kk is column kk*16 + g*8 + e
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < NKK / 2; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double th = rope_theta(theta_s, kk * 16 + g * 8 + e);
            float c, s;
            rope_cs(row0 + qb * 32 + l32, th, c, s);
            const float x1 = (float)qf[qb][kk][e], x2 = (float)qf[qb][kk + NKK / 2][e];
            qf[qb][kk][e] = (bf16)(x1 * c - x2 * s);
            qf[qb][kk + NKK / 2][e] = (bf16)(x2 * c + x1 * s);
          }
    }
    wait_vmem();
    __builtin_amdgcn_wave_barrier();
    if constexpr (ROPE) {
      // K in this wave's LDS tile: lane = row (rows past the sample end are zero)
      rope_rows_lds<D>(kt, theta_s, lane, row0 + lane);
      wait_lds();
      __builtin_amdgcn_wave_barrier();
    }

    // S^T[kb][qb]
    f32x16 sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = row_frag<D>(kt, kb * 32 + l32, kk, g);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = Elem<bf16>::mma(kf, qf[qb][kk], sacc[kb][qb]);
      }

    const int npad = 64 - r;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[kb][qb][i] *= a.scale_log2;
          mx = fmaxf(mx, sacc[kb][qb][i]);
        }
      mx = wave_xor32_max(mx);
      float ls = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = round_p<bf16>(exp2f(sacc[kb][qb][i] - mx));
          sacc[kb][qb][i] = e;
          ls += e;
        }
      // (a full block has no padded keys; its max may sit far below zero,
      // where 2^-m overflows and 0 * inf would be NaN)
      ls = wave_xor32_sum(ls) - (npad > 0 ? (float)npad * round_p<bf16>(exp2f(-mx)) : 0.0f);
      const float inv = 1.0f / ls;
      f32x16 oacc[ND];
#pragma unroll
      for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 pf = pack8_from(sacc[kb][qb], st * 8);
#pragma unroll
          for (int d = 0; d < ND; ++d) oacc[d] = Elem<bf16>::mma(tr_frag<D>(vt, kb, st, d * 32, lane), pf, oacc[d]);
        }
      const int row = qb * 32 + l32;
      if (row < r) {
        TO* orow = reinterpret_cast<TO*>(a.o) + qbase + (int64_t)row * HD;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            store4<TO>(orow + d * 32 + i4 * 8 + g * 4, oacc[d][i4 * 4] * inv, oacc[d][i4 * 4 + 1] * inv,
                       oacc[d][i4 * 4 + 2] * inv, oacc[d][i4 * 4 + 3] * inv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// backward: one wave pair per workgroup and per block
// ---------------------------------------------------------------------------
// A workgroup is one wave pair with its own worker list, so its barriers
// involve only the pair: two such workgroups fit in one CU's LDS and drift
// apart, and one pair's tile loads overlap the other's MFMA and softmax work.
constexpr int kPairThreads = 128;

template <typename TG, int D, bool ROPE = false>
__global__ __launch_bounds__(kPairThreads, 1) void block_bwd_kernel(BwdArgs a) {
  using T = Tile<D>;
  constexpr int NKK = D / 16, ND = D / 32;
  constexpr int PAIR_BYTES = 4 * T::BYTES + 2 * 64 * 4;
  static_assert(2 * (PAIR_BYTES + (ROPE ? D * 4 : 8)) <= 160 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(1024))) char smem[PAIR_BYTES];
  __shared__ double theta_s[ROPE ? D / 2 : 1];
  if constexpr (ROPE) {
    stage_theta<D>(theta_s, a.rope_theta);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, w2 = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  char* qt = smem;
  char* kt = qt + T::BYTES;
  char* vt = kt + T::BYTES;
  char* ot = vt + T::BYTES;  // dO
  float* L2s = reinterpret_cast<float*>(ot + T::BYTES);
  float* Dis = L2s + 64;
  const int worker = xcd_worker(blockIdx.x, gridDim.x);
  const int u_end = a.worker_off[worker + 1];
  const int HD = a.H * D;

  for (int u = a.worker_off[worker]; u < u_end; ++u) {
    const i32x4 unit = load_unit(a.units, u);
    const int b = unit[0], h = unit[1], t = unit[2];
    const Sample s = load_sample(a.samples, b);
    const int row0 = t * 64;
    const int r = min(64, s.lq - row0);
    const int64_t qbase = ((int64_t)(s.q0 + row0) * a.H + h) * D;
    const int64_t kbase = ((int64_t)(s.k0 + row0) * a.H + h) * D;
    {
      const uint32_t nbytes = (uint32_t)r * HD * 2;
      const rsrc_t rq = make_rsrc(reinterpret_cast<const bf16*>(a.q) + qbase, nbytes);
      const rsrc_t rk = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kbase, nbytes);
      const rsrc_t rv = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kbase, nbytes);
      const rsrc_t ro = make_rsrc(reinterpret_cast<const bf16*>(a.dout) + qbase, nbytes);
      load_tile_async<D>(qt, rq, 0, HD, lane, w2, 2);
      load_tile_async<D>(kt, rk, 0, HD, lane, w2, 2);
      load_tile_async<D>(vt, rv, 0, HD, lane, w2, 2);
      load_tile_async<D>(ot, ro, 0, HD, lane, w2, 2);
    }
    // the lane's angles (its row w2*32 + l32 is a query in phase 1 and a key
    // in phase 2, at one position), computed while the tiles are in flight,
    // rotate its share of the Q and K tiles once, then the dQ and dK rows in
    // the epilogues
    float rc[ROPE ? D / 4 : 1], rs[ROPE ? D / 4 : 1];
    if constexpr (ROPE) rope_lane_angles<D>(theta_s, row0 + w2 * 32 + l32, g, rc, rs);
    wait_vmem();
    __syncthreads();
    if constexpr (ROPE) {
      rope_lane_lds<D>(qt, w2 * 32 + l32, g, rc, rs);
      rope_lane_lds<D>(kt, w2 * 32 + l32, g, rc, rs);
      wait_lds();
      __syncthreads();
    }

    const int npad = 64 - r;
    // ---- phase 1: lane = query row (w2*32 + l32) ----
    {
      bf16x8 qf[NKK], of[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        qf[kk] = row_frag<D>(qt, w2 * 32 + l32, kk, g);
        of[kk] = row_frag<D>(ot, w2 * 32 + l32, kk, g);
      }
      f32x16 sacc[2], dpacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        dpacc[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sacc[kb] = Elem<bf16>::mma(row_frag<D>(kt, kb * 32 + l32, kk, g), qf[kk], sacc[kb]);
          dpacc[kb] = Elem<bf16>::mma(row_frag<D>(vt, kb * 32 + l32, kk, g), of[kk], dpacc[kb]);
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[kb][i] *= a.scale_log2;
          mx = fmaxf(mx, sacc[kb][i]);
        }
      mx = wave_xor32_max(mx);
      float ls = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = exp2f(sacc[kb][i] - mx);
          sacc[kb][i] = e;
          ls += e;
        }
      ls = wave_xor32_sum(ls) - (npad > 0 ? (float)npad * exp2f(-mx) : 0.0f);
      const float inv = 1.0f / ls;
      // Di = sum_j P_ij dP_ij over the block's keys (tail keys have dP = 0)
      float di = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[kb][i] *= inv;  // P
          di += sacc[kb][i] * dpacc[kb][i];
        }
      di = wave_xor32_sum(di);
      float ds[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[kb][i] = sacc[kb][i] * (dpacc[kb][i] - di);
      if (g == 0) {
        L2s[w2 * 32 + l32] = mx + __log2f(ls);
        Dis[w2 * 32 + l32] = di;
      }
      f32x16 dqacc[ND];
#pragma unroll
      for (int d = 0; d < ND; ++d) dqacc[d] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 df = pack8(&ds[kb][st * 8]);
#pragma unroll
          for (int d = 0; d < ND; ++d) dqacc[d] = Elem<bf16>::mma(tr_frag<D>(kt, kb, st, d * 32, lane), df, dqacc[d]);
        }
      const int row = w2 * 32 + l32;
      if constexpr (ROPE) rope_back_acc<ND>(dqacc, rc, rs);
      if (row < r) {
        TG* grow = reinterpret_cast<TG*>(a.dq) + qbase + (int64_t)row * HD;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            store4<TG>(grow + d * 32 + i4 * 8 + g * 4, dqacc[d][i4 * 4] * a.scale, dqacc[d][i4 * 4 + 1] * a.scale,
                       dqacc[d][i4 * 4 + 2] * a.scale, dqacc[d][i4 * 4 + 3] * a.scale);
      }
    }
    __syncthreads();

    // ---- phase 2: lane = key row (w2*32 + l32) ----
    {
      bf16x8 kf[NKK], vf[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        kf[kk] = row_frag<D>(kt, w2 * 32 + l32, kk, g);
        vf[kk] = row_frag<D>(vt, w2 * 32 + l32, kk, g);
      }
      f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        dkacc[d] = f32x16{};
        dvacc[d] = f32x16{};
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sacc = Elem<bf16>::mma(row_frag<D>(qt, qb * 32 + l32, kk, g), kf[kk], sacc);
          dpacc = Elem<bf16>::mma(row_frag<D>(ot, qb * 32 + l32, kk, g), vf[kk], dpacc);
        }
        float p[16], ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qb * 32 + acc_row(i, g);
          p[i] = exp2f(sacc[i] * a.scale_log2 - L2s[q]);
          ds[i] = p[i] * (dpacc[i] - Dis[q]);
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 pf = pack8(&p[st * 8]);
          const bf16x8 df = pack8(&ds[st * 8]);
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            dvacc[d] = Elem<bf16>::mma(tr_frag<D>(ot, qb, st, d * 32, lane), pf, dvacc[d]);
            dkacc[d] = Elem<bf16>::mma(tr_frag<D>(qt, qb, st, d * 32, lane), df, dkacc[d]);
          }
        }
      }
      const int row = w2 * 32 + l32;
      if constexpr (ROPE) rope_back_acc<ND>(dkacc, rc, rs);
      if (row < r) {
        TG* krp = reinterpret_cast<TG*>(a.dk) + kbase + (int64_t)row * HD;
        TG* vrp = reinterpret_cast<TG*>(a.dv) + kbase + (int64_t)row * HD;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int col = d * 32 + i4 * 8 + g * 4;
            store4<TG>(krp + col, dkacc[d][i4 * 4] * a.scale, dkacc[d][i4 * 4 + 1] * a.scale,
                       dkacc[d][i4 * 4 + 2] * a.scale, dkacc[d][i4 * 4 + 3] * a.scale);
            store4<TG>(vrp + col, dvacc[d][i4 * 4], dvacc[d][i4 * 4 + 1], dvacc[d][i4 * 4 + 2], dvacc[d][i4 * 4 + 3]);
          }
      }
    }
    __syncthreads();  // tiles are reloaded next round
  }
}

}  // namespace jattn
