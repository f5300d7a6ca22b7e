// Deep LDS rings for the persistent attention kernels on gfx950.
//
// A worker walks its units' steps in order; a producer cursor runs NS - 1 (or
// NS - 2) steps ahead of the consumer across unit boundaries and fills ring
// stages with buffer loads whose destination is LDS.  Vector memory
// operations of a wave complete in issue order (loads and stores share
// vmcnt), so the consumer waits only until the loads of the step it needs
// have landed: s_waitcnt vmcnt(n) with n = the operations this wave issued
// after them.  The ledger below keeps that count exact for the operations the
// kernel counts; operations it does not count (the compiler's own loads, an
// uncounted store) were issued later still, so they only make a wait
// stricter.  Nothing here may branch on lane-varying data around a counted
// operation: a wave that skipped one would wait too little.
//
// Plan records are read through scalar loads: addresses are wave-uniform and
// the data is read-only for the whole launch, so the constant address space
// applies.  Scalar loads are counted by lgkmcnt, which keeps the compiler from
// placing vmcnt waits (and with them waits on the whole ring) on plan reads.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "lds_tiles.hpp"

namespace jattn {

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

// s_waitcnt vmcnt(n) for a runtime n (clamped to 0..63 by the caller): binary
// dispatch to compile-time immediates.
template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID)
      wait_vmcnt_le<MID, HI>(n);
    else
      wait_vmcnt_le<LO, MID - 1>(n);
  }
}

// Number of the NI load instructions part, part + NP, ... that wave `part` issues.
__device__ __forceinline__ constexpr int loads_of(int NI, int part, int NP) {
  return part < NI ? (NI - part + NP - 1) / NP : 0;
}

// Per-wave count of the vector memory operations issued through a ring, and
// its value right after the loads of each of the last L productions (a
// production past the end of the worker's steps issues nothing and records
// the count unchanged).  With L productions in flight when a step is
// acquired, the acquired step is always the oldest of them.
//
// The wait uses one compile-time count N: in the steady state at least N
// operations follow the oldest production (N = the loads of the L - 1
// younger productions, taking the wave with the fewest), so vmcnt(N) is
// enough; when fewer follow (the last steps of the worker), vmcnt(0).  A
// wave that issued more than N after it waits a little longer than needed.
// One compare and branch instead of a dispatch over every possible count.
// N2 > N adds a second level for waves that also count stores between
// productions (N2 = N plus the stores of the steps in flight): without it
// every wait would also wait for those stores.
template <int L, int N, int N2 = 0>
struct VmLedger {
  static_assert(N >= 0 && N < 64 && N2 < 64, "vmcnt range");
  int issued = 0;
  int mark[L] = {};
  __device__ __forceinline__ void produced(int ops) {
    issued += ops;
#pragma unroll
    for (int i = L - 1; i > 0; --i) mark[i] = mark[i - 1];
    mark[0] = issued;
  }
  // operations issued outside a production that the waits may leave in flight
  __device__ __forceinline__ void counted(int ops) { issued += ops; }
  // wait until the loads of the oldest production in flight have landed
  __device__ __forceinline__ void wait_oldest() const {
    const int after = issued - mark[L - 1];
    if constexpr (N2 > N) {
      if (after >= N2) {
        wait_vmcnt<N2>();
        return;
      }
    }
    if constexpr (N == 0) {
      wait_vmcnt<0>();
    } else {
      if (after >= N)
        wait_vmcnt<N>();
      else
        wait_vmcnt<0>();
    }
  }
};

// Buffer descriptor words that walk a tensor step by step: base address and
// the bytes left from it.  LEFT64: the bytes left may exceed the 31-bit
// records range (clamped when the words are built); else they are below 2^31
// by construction (one sample's rows) and only clamped at zero.
template <bool LEFT64>
struct Walker {
  using L = typename std::conditional<LEFT64, int64_t, int32_t>::type;
  uint64_t addr;
  L left;
  __device__ __forceinline__ void start(const void* base, int64_t off, int64_t bytes_left) {
    addr = (uint64_t)(uintptr_t)base + (uint64_t)off;
    left = (L)bytes_left;
  }
  __device__ __forceinline__ void advance(int64_t bytes) {
    addr += (uint64_t)bytes;
    left -= (L)bytes;
  }
  __device__ __forceinline__ i32x4 words() const {
    int32_t n;
    if constexpr (LEFT64)
      n = left < 0 ? 0 : (left > 0x7fffffff ? 0x7fffffff : (int32_t)left);
    else
      n = left < 0 ? 0 : left;
    return i32x4{(int)(uint32_t)addr, (int)(uint32_t)(addr >> 32), n, 0x00020000};
  }
};

// Buffer stores of four consecutive output elements (one instruction each):
// offsets at or past the descriptor's records are dropped, so a lane without
// a valid row passes an out-of-range offset instead of branching, and the
// wave's count of issued operations stays independent of the data.
template <typename T>
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t voff, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void buf_store4<bf16>(rsrc_t r, uint32_t voff, float a, float b, float c, float d) {
  const bf16x2 lo = {(bf16)a, (bf16)b}, hi = {(bf16)c, (bf16)d};
  typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 v = {__builtin_bit_cast(int32_t, lo), __builtin_bit_cast(int32_t, hi)};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}
template <>
__device__ __forceinline__ void buf_store4<float>(rsrc_t r, uint32_t voff, float a, float b, float c, float d) {
  const i32x4 v = {(int32_t)__float_as_uint(a), (int32_t)__float_as_uint(b), (int32_t)__float_as_uint(c),
                   (int32_t)__float_as_uint(d)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}

}  // namespace jattn
