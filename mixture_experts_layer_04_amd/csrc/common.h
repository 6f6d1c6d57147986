// Device-side helpers shared by the libmoe kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger
// unsigned); used to reduce (key, id) pairs with one integer max.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Wave reductions on DPP row operations (quad xor 1, quad xor 2, half-row
// mirror, row mirror; afterwards every lane of a 16-lane row holds the row's
// result) and v_readlane of the four rows.  The order of operations is fixed
// (so sums are deterministic) and the result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  const int i = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(i, i, CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// every lane gets the max of its 16-lane row (the DPP steps of wave_max_u)
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  return fmaxf(v, dpp_f32<0x140>(v));
}
__device__ __forceinline__ float wave_max_u(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum_u(float v) {
  v = v + dpp_f32<0xB1>(v);
  v = v + dpp_f32<0x4E>(v);
  v = v + dpp_f32<0x141>(v);
  v = v + dpp_f32<0x140>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Last-workgroup elections: before the barrier that precedes one thread's
// agent-scope release, every wave that stored data the elected workgroup
// reads waits until its stores are complete (in the L2).  The barrier does
// not wait for them, and the one thread's release (L2 write-back, then its
// own wave's count) would otherwise miss stores of the other waves still in
// flight.
__device__ __forceinline__ void wait_wave_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Pair table entries of the paired GEMM tiles: the first block of the pair
// (bits 0-28), bit 30 when it holds two blocks, and two window bits.  The
// pairs of one expert form windows of two (its pairs 0 and 1, 2 and 3, ...;
// a last odd pair is a window of one): bit 29 marks the first pair of a
// window of two, bit 31 the second.  A window's N tiles run interleaved,
// (pair 0, n 0), (pair 1, n 0), (pair 0, n 1), ..., so the two tiles that
// read the same weight rows run side by side.
constexpr int32_t kPairTwo = 1 << 30;
constexpr int32_t kPairWinFirst = 1 << 29;
constexpr int32_t kPairWinSecond = (int32_t)0x80000000u;
constexpr int32_t kPairBlockMask = (1 << 29) - 1;
__device__ __forceinline__ int32_t pair_entry(int first_block, bool two, bool win_first, bool win_second) {
  return first_block | (two ? kPairTwo : 0) | (win_first ? kPairWinFirst : 0) | (win_second ? kPairWinSecond : 0);
}
struct PairTile {
  int blk;   // first block
  bool two;  // two blocks
  int nt;    // N tile
};
// Logical tile L (pair-major numbering: L / ntn is a pair, counted over the
// table's entries) of a table with ntn N tiles per pair, with each window's
// tiles interleaved.  A window of pairs [w, w + sz) owns the logical tiles
// [w ntn, (w + sz) ntn); tile w ntn + i is pair w + i % sz, N tile i / sz.
// npairs bounds the entries read (L < npairs ntn), also for a table whose
// window bits do not match its count.  WIN = false: plain pair-major order
// (the window bits are ignored).
template <bool WIN>
__device__ __forceinline__ PairTile pair_tile(const int32_t* pairs, int npairs, int64_t L, int ntn) {
  const int jj = (int)(L / ntn);
  const int32_t fw = __builtin_amdgcn_readfirstlane(pairs[1 + jj]);
  int w = jj, sz = 1;
  if (!WIN) {
    // nothing to do: one pair per window
  } else if ((fw & kPairWinFirst) && jj + 1 < npairs) {
    sz = 2;
  } else if ((fw & kPairWinSecond) && jj > 0) {
    w = jj - 1;
    sz = 2;
  }
  const int64_t local = L - (int64_t)ntn * w;
  const int entry = w + (int)(local % sz);
  const int32_t pe = entry == jj ? fw : __builtin_amdgcn_readfirstlane(pairs[1 + entry]);
  return PairTile{(int)(pe & kPairBlockMask), (pe & kPairTwo) != 0, (int)(local / sz)};
}

}  // namespace moe

// Launch-side helpers (host).
#define MOE_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;   \
  } while (0)

namespace moe {
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace moe
