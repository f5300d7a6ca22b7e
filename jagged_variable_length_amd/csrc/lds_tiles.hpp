// LDS tile helpers for gfx950: row-major bf16 tiles filled straight from HBM
// with buffer loads whose destination is LDS, XOR-swizzled 16-byte chunks,
// and transposed operand reads with ds_read_b64_tr_b16.
#pragma once
#include "common.hpp"

namespace jattn {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer descriptor as four SGPR words (base, size, raw 32-bit format) for
// the LDS-destination loads below.  Inputs are wave-uniform at every call.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4{(int)__builtin_amdgcn_readfirstlane((uint32_t)p), (int)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)),
               (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// LDS byte address of a pointer into a __shared__ array, as M0 and the ds_*
// instructions see it.  Taken once per kernel; stage and tile addresses are
// then plain 32-bit scalar offsets from it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}

// Descriptor moved `bytes_off` bytes forward with `records` bytes left
// (records <= 0 -> every load of it reads zero).  Records are capped below
// 2^31, so the 0x80000000 offset that marks a pad lane is always out of
// range.  Scalar arithmetic only.
__device__ __forceinline__ i32x4 rsrc_at(const i32x4& r, int64_t bytes_off, int64_t records) {
  const uint64_t p = ((uint64_t)(uint32_t)r[0] | ((uint64_t)(uint32_t)r[1] << 32)) + (uint64_t)bytes_off;
  const int64_t n = records < 0 ? 0 : (records > 0x7fffffff ? 0x7fffffff : records);
  return i32x4{(int)(uint32_t)p, (int)(uint32_t)(p >> 32), (int)(uint32_t)n, r[3]};
}

// HBM -> LDS loads (M0 = LDS byte address of the 64-lane group; lane l writes
// at M0 + 16*l, or the 4-byte slot M0 + 4*l for the dword and 2-byte forms,
// the 2-byte value zero-extended).  Issued as inline asm so that the compiler
// does not attach its own conservative vmcnt waits to unrelated LDS reads; the
// kernels wait for these loads explicitly (s_waitcnt vmcnt + barrier) before
// reading the data.  A write of M0 followed by an LDS-DMA load needs one wait
// state on this target (the compiler puts an s_nop between them for its own
// LDS-DMA loads; inline asm gets no hazard padding, so it is written here).
__device__ __forceinline__ void lds_dma16(const i32x4& r, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory");
}
__device__ __forceinline__ void lds_dma4(const i32x4& r, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory");
}
__device__ __forceinline__ void lds_dma2(const i32x4& r, uint32_t m0, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ushort %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory");
}

// Row-major tile of bf16 rows of D elements with PAD spare 16-byte slots per
// row (pitch = (D/8 + PAD) * 16 bytes).  The padding spreads consecutive rows
// over the LDS banks, and since addresses are row * pitch + column, every
// fragment of one lane is a fixed immediate offset from one base register.
// One load instruction fills 64 consecutive 16-byte slots; lanes that land on
// a pad slot load out of range (zero).
template <int D, int PAD>
struct PadTile {
  static constexpr int CPR = D / 8;      // 16-byte chunks of data per row
  static constexpr int SPR = CPR + PAD;  // slots per row
  static constexpr int PITCH = SPR * 16;
  template <int ROWS>
  static constexpr int ninst() { return (ROWS * SPR + 63) / 64; }
  template <int ROWS>
  static constexpr int bytes() { return ninst<ROWS>() * 1024; }
  static __device__ __forceinline__ int off(int r, int col) { return r * PITCH + col * 2; }
};

// Loads ROWS rows of one (sample, head) into a PadTile, the load instructions
// dealt round-robin over NPARTS waves.  The per-lane source offsets depend
// only on the row pitch in HBM (H*D elements), so they are computed once; a
// step only moves the scalar descriptor (rsrc_at) to its first row, and rows
// at or past the descriptor end arrive as zeros.
// PERM: tile row m of every 32-row block holds source row perm32(m) of that
// block.  Read as an MFMA A operand in tile order, such a tile makes the
// accumulator of lane half g hold rows 16g .. 16g+15 of the block in slot
// order (perm32(acc_row(i, g)) = 16g + i), and the transposed reads in
// accumulator order (trans_frag) deliver source rows in plain order.
template <int D, int PAD, int ROWS, int NPARTS, bool PERM = false>
struct RowLoader {
  using T = PadTile<D, PAD>;
  static constexpr int NI = T::template ninst<ROWS>();
  static constexpr int NJ = (NI + NPARTS - 1) / NPARTS;
  uint32_t voff[NJ];
  __device__ __forceinline__ void init(int part, int lane, int HD) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int slot = (part + j * NPARTS) * 64 + lane;
      const int rr = slot / T::SPR, ch = slot % T::SPR;
      const int src = PERM ? ((rr & ~31) | perm32(rr & 31)) : rr;
      voff[j] = (ch < T::CPR && rr < ROWS) ? (uint32_t)(src * HD + ch * 8) * 2 : 0x80000000u;
    }
  }
  // part must be wave-uniform; tile is the LDS byte address of the tile
  __device__ __forceinline__ void issue(uint32_t tile, const i32x4& r, int part) const {
#pragma unroll
    for (int j = 0; j < NJ; ++j) issue_one(j, tile, r, part);
  }
  // the j-th load of this part (j a compile-time constant after unrolling)
  __device__ __forceinline__ void issue_one(int j, uint32_t tile, const i32x4& r, int part) const {
    const int inst = part + j * NPARTS;
    if (NI % NPARTS == 0 || inst < NI) lds_dma16(r, tile + inst * 1024, voff[j]);
  }
};

// Bias tile: ROWS rows x COLS keys of one (sample, head) bias block, whose
// rows are lk elements apart in HBM at any 2-byte alignment.  Each row is
// moved as COLS/8 unaligned 16-byte loads (the code-object ABI of this
// target runs with unaligned buffer access enabled, and the range check is
// per dword) into a PadTile<COLS, PAD>, so the tile holds plain bf16 rows at
// 16-byte aligned positions.  Loads past the descriptor end read as zero;
// keys at or past lk carry the next row's values and are masked by the
// kernels.  The offsets depend on lk, so they are rebuilt per unit.
template <int COLS, int PAD, int ROWS, int NPARTS>
struct BiasLoader {
  using T = PadTile<COLS, PAD>;
  static constexpr int NI = T::template ninst<ROWS>();
  static constexpr int NJ = (NI + NPARTS - 1) / NPARTS;
  uint32_t voff[NJ];
  __device__ __forceinline__ void init(int part, int lane, int lk) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int slot = (part + j * NPARTS) * 64 + lane;
      const int rr = slot / T::SPR, ch = slot % T::SPR;
      voff[j] = (ch < T::CPR && rr < ROWS) ? (uint32_t)(rr * lk + ch * 8) * 2 : 0x80000000u;
    }
  }
  __device__ __forceinline__ void issue(uint32_t tile, const i32x4& r, int part) const {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int inst = part + j * NPARTS;
      if (NI % NPARTS == 0 || inst < NI) lds_dma16(r, tile + inst * 1024, voff[j]);
    }
  }
  // Same, with tile rows at or past `rows` read as zero.
  __device__ __forceinline__ void issue_rows(uint32_t tile, const i32x4& r, int part, int lane, int rows) const {
#pragma unroll
    for (int j = 0; j < NJ; ++j) issue_one_rows(j, tile, r, part, lane, rows);
  }
  __device__ __forceinline__ void issue_one_rows(int j, uint32_t tile, const i32x4& r, int part, int lane,
                                                 int rows) const {
    const int inst = part + j * NPARTS;
    const int rr = (inst * 64 + lane) / T::SPR;
    if (NI % NPARTS == 0 || inst < NI) lds_dma16(r, tile + inst * 1024, rr < rows ? voff[j] : 0x80000000u);
  }
};

// Eight consecutive bf16 (one aligned 16-byte LDS read) widened to fp32.
__device__ __forceinline__ void bf16x8_to_f32(const char* p, float* out) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(w[j] << 16);
    out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

// B/A fragment of a row operand: 8 bf16 of row `row`, columns kk*16 + g*8 ..
template <int D, int PAD>
__device__ __forceinline__ bf16x8 rows_frag(const char* tile, int row, int kk, int g) {
  return *reinterpret_cast<const bf16x8*>(tile + PadTile<D, PAD>::off(row, kk * 16 + g * 8));
}

// A fragment of X^T for MFMA 32x32x16: lane l gets X[rows][col0 + l%32] for the
// 8 rows that accumulator block `blk`, step `st` assigns to lane half g
// (rows blk*32 + 16st + 4g + 0..3 and +8..+11).  Uses ds_read_b64_tr_b16:
// within each 16-lane group, lane i receives element i%4 of the 8-byte
// pieces addressed by lanes i/4 + 4k, so lane j addresses row base + j/4,
// columns col0 + 4*(j%4) .. +3.
template <int D, int PAD>
__device__ __forceinline__ bf16x8 trans_frag(const char* tile, int blk, int st, int col0, int lane) {
  const int i = lane & 15, grp = (lane >> 4) & 1, g = lane >> 5;
  const int col = col0 + 16 * grp + 4 * (i & 3);
  const int r1 = blk * 32 + 16 * st + 4 * g + (i >> 2);
  v4i16_t lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
#if __HIP_DEVICE_COMPILE__
  lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + PadTile<D, PAD>::off(r1, col)));
  hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + PadTile<D, PAD>::off(r1 + 8, col)));
#endif
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ void wait_vmcnt0() {
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 pack8v(const f32x16& v, int off) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)v[off + j];
  return r;
}

}  // namespace jattn
