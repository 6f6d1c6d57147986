// Grouped expert GEMMs for every weight format: GEMM1 (+ SwiGLU epilogue,
// + requantisation for the fp8 formats) and GEMM2, plus the activation
// quantisation of x.
//
// [Kernels] "The fused expert GEMM": each tile owns one block of BLOCK_M rows
// and that block's single expert from the block table; activation rows are
// gathered through sorted_ids / k (rows at or past T*k are padding and
// contribute zeros); gate and up columns give silu(g) * u in the epilogue
// ([MegaMoE] §3.5: activation and requantisation are the tail of the GEMM1
// task).  GEMM2 reads the SwiGLU rows in block order and writes each real
// row to its assignment slot of the [T*k, H] output.
//
// Formats (weights w13 [E, 2F, H], w2 [E, H, F], K contiguous):
//  * BF16:  v_mfma_f32_16x16x32_bf16.
//  * FP8:   e4m3 x e4m3 on v_mfma_f32_16x16x128_f8f6f4; one MFMA spans one
//           128-wide K block, so its result is scaled by the activation
//           row's fp32 scale and the weight block's fp32 scale and added to
//           the accumulator ([Kernels] "Combine, backward and low precision":
//           1x128 activation tiles, 128x128 weight blocks).  The SwiGLU
//           output is requantised per row per 128 columns (scale amax/448).
//  * MX:    e4m3 activations x e2m1 weights on
//           v_mfma_scale_f32_16x16x128_f8f6f4 with e8m0 scales per 32 K
//           applied by the instruction ([MegaMoE] §1.1); the SwiGLU output
//           is requantised per row per 32 columns with the power-of-two
//           scale pow2_at_least(amax/448) ([MegaMoE] §3.5).
//
// Operand layouts inside one MFMA (lane l: row / column l % 16, group
// g = l / 16; measured on gfx950):
//  * bf16 16x16x32: 8 values at K = 8g .. 8g+7 of the 32-wide step;
//  * 8-bit 16x16x128: 32 bytes, K = 16g .. 16g+15 then 64+16g .. 64+16g+15;
//  * 4-bit 16x16x128: 32 nibbles at K = 32g .. 32g+31, low nibble first;
//  * the e8m0 scale of 32-wide K block b for row / column i is read from
//    lane 16b + i;
//  * the 16x16 fp32 result: lane l holds rows 4g .. 4g+3 of column l % 16.
//
// Two tile families:
//  * BLOCK_M = 16 ("stream", decode): the weights are the traffic.  Small
//    tiles (16 or 32 weight rows) spread the weight bytes evenly over the
//    CUs; the 8 waves of a workgroup split K, each loading several MFMA
//    steps of operands straight into VGPRs before multiplying them (a weight
//    element is used once); the partial tiles are added in LDS in a fixed
//    order.  For FP8 / MX the fp32 SwiGLU rows are requantised by a second,
//    row-parallel kernel.
//  * BLOCK_M >= 32 ("tiled", prefill): 2 x 2 waves, A (BLOCK_M rows) and B
//    tiles copied straight into a 3-stage LDS ring two K steps (128 bytes of
//    K per row each) ahead of the multiply; one barrier per step; the output
//    tile leaves through LDS as whole rows.
// Tiles are visited in a grid-stride loop bounded by the padded length read
// on the device (no workgroup is launched for blocks that do not exist),
// block-major: an XCD takes a contiguous run of blocks and all of their N
// tiles, so a block's A rows are read from HBM once and the weight tiles of
// an expert are reused by its following blocks.

#include <atomic>
#include <cmath>

#include "common.h"
#include "launch.h"
#include "quant.h"

namespace moe {

namespace {

enum Fmt { F_BF16 = 0, F_FP8 = 1, F_MX = 2 };

struct GemmP {
  const uint8_t* x;       // GEMM1 A source: bf16 x [T, H] or e4m3 xq [T, H]
  const void* xs;         // x scales: fp32 [T, H/128] (FP8) or e8m0 [T, H/32] (MX)
  const uint8_t* w13;
  const void* w13_s;
  const uint8_t* w2;
  const void* w2_s;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* npp;
  uint8_t* act;           // [max_padded, F] bf16 or e4m3
  void* act_s;            // fp32 [max_padded, F/128] (FP8) or e8m0 [max_padded, F/32] (MX)
  float* act32;           // BLOCK_M 16, FP8 / MX: fp32 SwiGLU rows [max_padded, F]
  uint16_t* out;          // [T*k, H] bf16
  const int32_t* pairs;   // paired tiled kernel: pair table (pair_table_kernel)
  int* queue;             // tiled kernels: 8 XCD tile counters + done count, zero on entry and exit
  float lim;              // SwiGLU clamp (+inf: none)
  int H, F, k, A;
};

template <int F>
struct Tr;
template <>
struct Tr<F_BF16> {
  static constexpr int AB = 2;         // bytes per A element
  static constexpr int KSTEP = 64;     // K elements per 128-byte step
  static constexpr int BROW = 128;     // B bytes per row per step
  static constexpr int BNA_STREAM = 16;
};
template <>
struct Tr<F_FP8> {
  static constexpr int AB = 1;
  static constexpr int KSTEP = 128;
  static constexpr int BROW = 128;
  static constexpr int BNA_STREAM = 128;
};
template <>
struct Tr<F_MX> {
  static constexpr int AB = 1;
  static constexpr int KSTEP = 128;    // per MFMA step; the tiled kernel can take KMX = 2 of them per K step
  static constexpr int BROW = 64;
  static constexpr int BNA_STREAM = 32;
};

// MFMA operand types and K per instruction of each format.
template <int F>
struct SOp;
template <>
struct SOp<F_BF16> {
  using A = bf16x8_t;
  using B = bf16x8_t;
  static constexpr int SK = 32;  // K elements per MFMA step
  static constexpr int S = 8;    // steps loaded at once
};
template <>
struct SOp<F_FP8> {
  using A = i32x8_t;
  using B = i32x8_t;
  static constexpr int SK = 128;
  static constexpr int S = 4;
};
template <>
struct SOp<F_MX> {
  using A = i32x8_t;
  using B = i32x4_t;
  static constexpr int SK = 128;
  static constexpr int S = 4;
};

// silu(min(g, lim)) * clamp(u, -lim, lim) ([MegaMoE] §3.5); lim = +inf: no
// clamp.  silu(g) = g / (1 + e^-g) on the hardware exp2 and reciprocal
// (about 1 ulp each; e^-g overflows to +inf for g < -88, giving -0 * u)
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f)) * u;
}
__device__ __forceinline__ float swiglu(float g, float u, float lim) {
  return silu_mul(fminf(g, lim), fminf(fmaxf(u, -lim), lim));
}
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Rows of a staged GEMM2 output tile (bf16, CH 16-byte chunks per row, LDS
// row stride CH * 16) to their assignment slots in out [T*k, H]: thread t
// stores chunk t % CH of rows t / CH + (NT / CH) i.  load_slots fetches the
// slots of the thread's rows all at once (one memory latency instead of one
// per row); call it before staging the tile so that the latency overlaps.
template <int NT, int CH, int ROWS>
struct RowScatter {
  static constexpr int RP = NT / CH;      // rows per pass
  static constexpr int NP = ROWS / RP;    // passes over ROWS rows
  static_assert(NT % CH == 0 && ROWS % RP == 0, "whole passes");
  int sid[NP];
  __device__ __forceinline__ void load_slots(const GemmP& p, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int lr = tid / CH + RP * i;
      sid[i] = lr < nrows ? p.sorted_ids[row0 + lr] : p.A;
    }
  }
  __device__ __forceinline__ void store(const GemmP& p, const uint8_t* st, int col0, int tid) const {
    const int c = tid % CH;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (sid[i] >= p.A) continue;  // padding, or past the tile's rows
      const int lr = tid / CH + RP * i;
      const uint4 val = *reinterpret_cast<const uint4*>(st + lr * CH * 16 + c * 16);
      // non-temporal: the combine reads these rows once, later; the L2 keeps
      // the GEMM's own operands instead (DSV4 T=8192 layer about 7 us faster)
      __builtin_nontemporal_store(u32x4_t{val.x, val.y, val.z, val.w},
                                  reinterpret_cast<u32x4_t*>(p.out + (size_t)sid[i] * p.H + col0 + c * 8));
    }
  }
};

// ---------------------------------------------------------------------------
// Activation quantisation of x (FP8: per 128, fp32 scale amax/448;
// MX: per 32, e8m0 scale pow2_at_least(amax/448)).  One workgroup per token,
// each thread 8 consecutive values.
template <int F>
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t* x, uint8_t* xq, void* xs, int H) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)t * H + h);
    float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    constexpr int GL = (F == F_FP8) ? 16 : 4;  // lanes per scale group
#pragma unroll
    for (int off = 1; off < GL; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    float g[8];
    if (F == F_FP8) {
      const float s = fp8_group_scale(m);
      if ((lane & 15) == 0) static_cast<float*>(xs)[(size_t)t * (H / 128) + h / 128] = s;
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = fp8_scaled(f[i], s);
    } else {
      const uint32_t c = mx_group_code(m);
      const float inv = e8m0_inv(c);
      if ((lane & 3) == 0) static_cast<uint8_t*>(xs)[(size_t)t * (H / 32) + h / 32] = (uint8_t)c;
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = clamp448(f[i] * inv);
    }
    uint2 q;
    q.x = pack4_e4m3(g[0], g[1], g[2], g[3]);
    q.y = pack4_e4m3(g[4], g[5], g[6], g[7]);
    *reinterpret_cast<uint2*>(xq + (size_t)t * H + h) = q;
  }
}

// ---------------------------------------------------------------------------
// MFMA operand loads from a row pointer (global or LDS).  `p` points at the
// row's first byte of the 128-byte (bf16: one 32-wide sub-step uses 64 of
// them) K step.
__device__ __forceinline__ bf16x8_t ld_bf16_op(const uint8_t* row, int ks, int g) {
  return *reinterpret_cast<const bf16x8_t*>(row + ks * 64 + g * 16);
}
__device__ __forceinline__ i32x8_t ld_f8_op(const uint8_t* row, int g) {
  const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(row + g * 16);
  const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(row + 64 + g * 16);
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ i32x8_t ld_f4_op(const uint8_t* row, int g) {
  const i32x4_t v = *reinterpret_cast<const i32x4_t*>(row + g * 16);
  return i32x8_t{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
}
__device__ __forceinline__ f32x4_t mfma_f8(const i32x8_t& a, const i32x8_t& b) {
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_mx(const i32x8_t& a, const i32x8_t& b, f32x4_t c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

// Per-tile row bookkeeping: the A row source (token row for GEMM1, padded row
// for GEMM2) of a row of the tile.
template <bool G1>
__device__ __forceinline__ int a_row_index(const GemmP& p, int blk, int bm, int row, bool& valid) {
  if (G1) {
    const int sid = p.sorted_ids[blk * bm + row];
    valid = sid < p.A;
    return valid ? sid / p.k : 0;
  }
  valid = true;
  return blk * bm + row;
}

// ---------------------------------------------------------------------------
// Tiled kernel.  Tile: BM rows x BNW weight rows (GEMM1: BNW/2 gate rows then
// the matching BNW/2 up rows = BNW/2 SwiGLU columns; GEMM2: BNW output
// columns).  NW waves as 2 x WN (WN = NW / 2): wave (wm, wn) owns rows
// [wm*BM/2, +BM/2) and weight rows: GEMM1 gate [wn*BNW/(2 WN), +BNW/(2 WN))
// and the matching up rows BNW/2 further; GEMM2 [wn*BNW/WN, +BNW/WN).
//
// K steps of 128 bytes per row are copied global -> LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging) into a ring of NS stages, NS - 1
// steps ahead of the multiply; one barrier per step.  Inside a stage a row's
// 16-byte chunk c sits at slot c ^ f(row) (f(row) = (row / (16 / chunks per
// row)) mod chunks per row), so the 16 rows one MFMA operand read touches
// fall in 16 different bank groups.  The epilogue stages the output tile in
// LDS and writes whole rows with 16-byte stores.
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// 4-byte copy of a scale word (flat address)
__device__ __forceinline__ void g2lds4(const void* g, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((gvoid_t*)g, (lvoid_t*)lds_dst, 4, 0, 0);
}
// 16-byte tile copies use the buffer-resource form: a per-lane 32-bit byte
// offset, a wave-uniform offset (the K step) and a 4-dword descriptor of the
// source range (reads at or past `bytes` return zero).  Unlike the
// flat-address form it lets the compiler keep counting the LDS reads in
// flight precisely instead of waiting for all of them, and the step offset
// costs no vector instruction.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}
__device__ __forceinline__ void buf2lds16(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lvoid_t*)lds_dst, 16, voff, soff, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// vmcnt(clamp(n, LO, HI)) for a wave-uniform n, by bisection (the count is an
// immediate of the instruction)
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_in(int n) {
  if constexpr (LO == HI) {
    wait_vm<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vm_in<MID, HI>(n);
    else wait_vm_in<LO, MID - 1>(n);
  }
}
// vmcnt(min(n, N)) for a wave-uniform n >= 0
template <int N>
__device__ __forceinline__ void wait_vm_upto(int n) {
  wait_vm_in<0, N>(n);
}
// Copy instructions a wave has issued after the last one of step s when it
// waits ahead of step s, for a stream of L copy instructions per step issued
// D steps ahead (step u's copies at step u - D, the first D steps before step
// 0) with one scale-group copy right after step u's copies when u is a
// multiple of SCG (group u / SCG + 1, if it exists): the copies of steps
// s + 1 .. s + D - 1 that exist, and the scale groups issued at steps
// max(s - D, 0) .. s - 1.  Copies complete in issue order, so leaving that
// many in flight means step s's have landed; memory operations issued after
// a tile's first copies (the previous tile's stores) only make it stricter.
template <int L, int D, int SCG>
__device__ __forceinline__ int copies_after(int s, int nk, int ng) {
  int n = L * (min(s + D - 1, nk - 1) - s);
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int u = s - D + i;
    if (u >= 0 && u % SCG == 0 && u / SCG + 1 < ng) ++n;
  }
  return n;
}
// Workgroup barrier for the copy pipeline: each wave has already waited for
// its own copies of the step (wait_vm), so no memory fence is needed, and a
// fence would also wait for the copies still in flight for later steps.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// A barrier after which every wave sees the LDS writes made before it, with
// no wait on vector memory operations (copies into LDS and global stores stay
// in flight, unlike __syncthreads())
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), no other count
  barrier_no_fence();
}
typedef __attribute__((address_space(3))) int lds_int_t;
// the LDS byte address of a pointer into the workgroup's LDS
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Two 16-byte LDS reads, at byte address addr and addr + OFF, waited for in
// the same instruction group.  Reads the compiler sees after copies into LDS
// (buffer_load ... lds) are preceded by a wait for every such copy in flight
// when it cannot tell the addresses apart; these are not.  Only for LDS that
// no copy in flight writes.
template <int OFF>
__device__ __forceinline__ void lds_read2_b128(uint32_t addr, u32x4_t& a, u32x4_t& b) {
  static_assert(OFF > 0 && OFF < 65536, "offset");
  asm volatile(
      "ds_read_b128 %0, %2\n"
      "ds_read_b128 %1, %2 offset:%3\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b)
      : "v"(addr), "n"(OFF)
      : "memory");
}
template <int CPR>
__device__ __forceinline__ int swz(int c, int row) {
  return c ^ ((row / (16 / CPR)) & (CPR - 1));
}

// Slot of B chunk c of tile row rr: 128-byte rows as the A rows; 64-byte
// rows (MX with one MFMA step per K step) c ^ (rr / 2 % 4) (measured on
// gfx950: with it a fragment read of 16 rows hits no LDS bank twice, with
// c ^ (rr / 4 % 4) it did)
template <int CPRB>
__device__ __forceinline__ int bswz(int c, int rr) {
  return CPRB == 8 ? swz<8>(c, rr) : c ^ ((rr >> 1) & 3);
}

template <int F, bool G1, int BM, int BNW, int NS, int NW, int KMX>
__global__ __launch_bounds__(64 * NW) void gemm_tiled(GemmP p) {
  using T = Tr<F>;
  // fp8 at 64 and 128 rows skips padding fragments (measured, DSV3 T=2048
  // at 128 rows: layer 2496 -> 2400 us warm; at 32 rows, and for MX, no
  // gain: DSV3 T=256 level, DSV4 T=512 757 -> 769 us)
  constexpr bool SKIP_PAD = F == F_FP8 && BM >= 64;
  // MX with KMX = 2: a K step holds two 128-K MFMA steps, so a weight row's
  // step is a whole 128-byte line (a CU keeps a fixed number of copy
  // requests in flight, so full lines copy faster); the A rows (256 bytes)
  // sit in two 128-byte planes, one per MFMA step, with two scale words
  // per row
  constexpr int KSQ = (F == F_MX) ? KMX : 1;  // MFMA steps per K step (FP8 / MX)
  constexpr int APL = KSQ;                    // A planes
  constexpr int BROW = T::BROW * KSQ;         // B bytes per row and step
  constexpr int KSTEP = T::KSTEP * KSQ;
  constexpr int CPRB = BROW / 16;             // 16-byte chunks per B row and step
  constexpr int ASZ = APL * BM * 128;
  constexpr int BSZ = BNW * BROW;
  constexpr int WN = NW / 2;           // waves: 2 along M x WN along N
  constexpr int NT = 64 * NW;          // threads
  constexpr int FM = BM / 32;
  constexpr int FN = BNW / WN / 16;
  constexpr int LA = APL * BM * 8 / NT;  // A copy instructions per wave per step
  constexpr int LB = BNW * CPRB / NT;  // B copy instructions per wave per step
  static_assert(LA >= 1 && LB >= 1 && (!G1 || FN % 2 == 0), "tile too small for the wave count");
  // scales (FP8, MX): one 4-byte word per tile row and MFMA step (A: the
  // row's scale(s), B: the weight row's) copied with the data, MFMA step w
  // in scale plane w; every wave issues the same number of copies, the slots
  // past BM + BNW are never read
  constexpr int LSC1 = (F == F_BF16) ? 0 : (BM + BNW + NT - 1) / NT;  // copies per plane
  constexpr int LSC = LSC1 * KSQ;
  constexpr int SCPL = LSC1 * NT * 4;  // bytes per scale plane
  constexpr int LS = LA + LB + LSC;
  constexpr int SCSZ = SCPL * KSQ;
  constexpr int SSZ = ASZ + BSZ + SCSZ;
  constexpr int D = NS - 1;            // steps in flight ahead of the multiply
  static_assert(LS * (D > 1 ? D - 1 : 1) <= 63, "vmcnt range");
  static_assert(NS * SSZ <= 163840, "the ring must fit in LDS");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int K = G1 ? p.H : p.F;
  const int N = G1 ? p.F : p.H;
  const int BNO = G1 ? BNW / 2 : BNW;
  const int ntn = N / BNO;
  const int nblk = *p.npp / BM;
  const int64_t n_valid = (int64_t)nblk * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int nk = K / KSTEP;
  const int rowbytes_a = K * T::AB;
  const int rowbytes_b = (F == F_MX) ? K / 2 : K * T::AB;
  const uint8_t* asrc = G1 ? p.x : p.act;
  const uint8_t* wsrc = G1 ? p.w13 : p.w2;
  const size_t erows = G1 ? (size_t)2 * p.F : (size_t)p.H;
  // A source: the T token rows (GEMM1) or the padded rows (GEMM2)
  const rsrc_t ra = make_rsrc(asrc, (uint64_t)(G1 ? p.A / p.k : nblk * BM) * rowbytes_a);

  // tile-local weight row of fragment fn of this wave
  auto frag_lrow = [&](int fn) {
    return G1 ? (fn < FN / 2 ? wn * (BNW / (2 * WN)) + fn * 16 : BNW / 2 + wn * (BNW / (2 * WN)) + (fn - FN / 2) * 16)
              : wn * (BNW / WN) + fn * 16;
  };
  auto weight_row = [&](int nt, int lrow) {
    if (G1) return lrow < BNW / 2 ? nt * (BNW / 2) + lrow : p.F + nt * (BNW / 2) + (lrow - BNW / 2);
    return nt * BNW + lrow;
  };

  // Tiles: XCD x (workgroups are dealt to the XCDs round-robin) owns the
  // contiguous run [x per, x per + per) of logical tiles.  A workgroup's
  // first tile is its index among the XCD's workgroups; when the XCD has
  // more tiles than workgroups, each takes the next one from the XCD's
  // counter when it is done with the last, so the CUs of an XCD end within
  // one tile of each other.  The index goes through the first LDS word
  // while the ring is idle.
  const int xcd = blockIdx.x & 7;
  const int wpx = (int)(gridDim.x >> 3);  // workgroups per XCD
  const bool dyn = per > wpx;
  int j = (int)(blockIdx.x >> 3);
  for (;; ) {
    const int64_t L = (int64_t)xcd * per + j;
    if (j >= per || L >= n_valid) break;
    // block-major: the N tiles of a block follow each other (its A rows stay
    // in the L2 for all of them; the weight tiles are shared with the
    // expert's next blocks through the last-level cache)
    const int blk = (int)(L / ntn);
    const int nt = (int)(L % ntn);
    // uniform; readfirstlane keeps the weight descriptor in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(p.block_expert[blk]);
    // the valid rows of a block are a prefix of it (the alignment pads the
    // end of each expert's run): this wave's 16-row fragments past the last
    // valid row hold padding alone and are not multiplied
    int nf = FM;
    if constexpr (SKIP_PAD) {
      const int sid = lane < FM ? p.sorted_ids[blk * BM + wm * (BM / 2) + 16 * lane] : p.A;
      nf = __builtin_amdgcn_readfirstlane(__popcll(__ballot(sid < p.A)));
    }

    // per-lane source offsets of the copy instructions (the K step is added
    // as a uniform offset)
    // copy i: A plane i % APL, rows wave * BM / NW + 8 (i / APL) ..
    uint32_t ag[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = wave * (BM / NW) + 8 * (i / APL) + (lane >> 3);
      bool v;
      const int src = a_row_index<G1>(p, blk, BM, row, v);  // padding rows read token 0; never used
      ag[i] = (uint32_t)src * rowbytes_a + 128 * (i % APL) + 16 * swz<8>(lane & 7, row);
    }
    const rsrc_t rb = make_rsrc(wsrc + (size_t)e * erows * rowbytes_b, (uint64_t)erows * rowbytes_b);
    uint32_t bg[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = (wave * LB + i) * (64 / CPRB) + lane / CPRB;
      bg[i] = (uint32_t)weight_row(nt, row) * rowbytes_b + 16 * bswz<CPRB>(lane % CPRB, row);
    }
    // scale words: copy i fills plane i / LSC1, slot q = ((i % LSC1) * NW +
    // wave) * 64 + lane; q < BM: A row q, q < BM + BNW: B row q - BM.  Per
    // step the source advances by sc_step bytes.
    const uint8_t* scg[LSC > 0 ? LSC : 1];
    int sc_step[LSC > 0 ? LSC : 1];
    if (F != F_BF16) {
      const int kblocks = K / 128;  // FP8: one fp32 scale per 128 K; MX: 4 e8m0 per 128 K
#pragma unroll
      for (int i = 0; i < LSC; ++i) {
        const int q = ((i % LSC1) * NW + wave) * 64 + lane;
        const int pl = i / LSC1;
        if (q < BM) {
          bool v;
          const int src = a_row_index<G1>(p, blk, BM, q, v);
          if (F == F_FP8) {
            scg[i] = static_cast<const uint8_t*>(G1 ? p.xs : p.act_s) + ((size_t)src * kblocks) * 4;
            sc_step[i] = 4;
          } else {
            scg[i] = static_cast<const uint8_t*>(G1 ? p.xs : p.act_s) + (size_t)src * (K / 32) + 4 * pl;
            sc_step[i] = 4 * KSQ;
          }
        } else {
          const int lrow = q < BM + BNW ? q - BM : 0;
          const int wr = weight_row(nt, lrow);
          if (F == F_FP8) {
            scg[i] = static_cast<const uint8_t*>(G1 ? p.w13_s : p.w2_s) +
                     (((size_t)e * (erows / 128) + wr / 128) * kblocks) * 4;
            sc_step[i] = 4;
          } else {
            scg[i] = static_cast<const uint8_t*>(G1 ? p.w13_s : p.w2_s) + ((size_t)e * erows + wr) * (K / 32) + 4 * pl;
            sc_step[i] = 4 * KSQ;
          }
        }
      }
    }
    // copy step s into ring slot `slot`
    auto issue = [&](int s, int slot) {
      uint8_t* st = lds + slot * SSZ;
#pragma unroll
      for (int i = 0; i < LA; ++i)
        buf2lds16(ra, ag[i], s * 128 * APL, st + (i % APL) * BM * 128 + (wave * (BM / NW) + 8 * (i / APL)) * 128);
#pragma unroll
      for (int i = 0; i < LB; ++i) buf2lds16(rb, bg[i], s * BROW, st + ASZ + (wave * LB + i) * (64 / CPRB) * BROW);
#pragma unroll
      for (int i = 0; i < LSC; ++i)
        g2lds4(scg[i] + (size_t)s * sc_step[i], st + ASZ + BSZ + (i / LSC1) * SCPL + ((i % LSC1) * NW + wave) * 256);
    };

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Operand fragments of one MFMA sub-step, read from a ring slot.  BF16
    // has two 32-wide sub-steps per 64-element step, MX two 128-wide ones per
    // 256-element step, FP8 one.
    struct Frag {
      typename SOp<F>::A af[FM];
      typename SOp<F>::B bfr[FN];
      float as_[FM][4];  // FP8: A scales of the C rows
      float wsc[FN];     // FP8: weight block scales
      int sa[FM];        // MX: A e8m0
      int sb[FN];        // MX: weight e8m0
    };
    auto rd = [&](int s, int ks, Frag& f) {
      const uint8_t* Bs = lds + (s % NS) * SSZ + ASZ;
      const uint8_t* As = lds + (s % NS) * SSZ + (F == F_MX ? ks * BM * 128 : 0);
      const uint8_t* Ss = Bs + BSZ + (F == F_MX ? ks * SCPL : 0);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int rr = wm * (BM / 2) + fm * 16 + r;
        if constexpr (F == F_BF16) {
          f.af[fm] = *reinterpret_cast<const bf16x8_t*>(As + rr * 128 + 16 * swz<8>(ks * 4 + g, rr));
        } else {
          const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(As + rr * 128 + 16 * swz<8>(g, rr));
          const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(As + rr * 128 + 16 * swz<8>(4 + g, rr));
          f.af[fm] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          if constexpr (F == F_FP8) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              f.as_[fm][q] = reinterpret_cast<const float*>(Ss)[wm * (BM / 2) + fm * 16 + 4 * g + q];
          } else {
            f.sa[fm] = (int)Ss[rr * 4 + g];
          }
        }
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int rr = frag_lrow(fn) + r;
        if constexpr (F == F_BF16) {
          f.bfr[fn] = *reinterpret_cast<const bf16x8_t*>(Bs + rr * 128 + 16 * swz<8>(ks * 4 + g, rr));
        } else if constexpr (F == F_FP8) {
          const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(Bs + rr * 128 + 16 * swz<8>(g, rr));
          const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(Bs + rr * 128 + 16 * swz<8>(4 + g, rr));
          f.bfr[fn] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          f.wsc[fn] = reinterpret_cast<const float*>(Ss)[BM + frag_lrow(fn)];
        } else {
          f.bfr[fn] = *reinterpret_cast<const i32x4_t*>(Bs + rr * BROW + 16 * bswz<CPRB>(ks * 4 + g, rr));
          f.sb[fn] = (int)Ss[(BM + rr) * 4 + g];
        }
      }
    };
    auto mm = [&](const Frag& f) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (SKIP_PAD && fm >= nf) break;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          if constexpr (F == F_BF16) {
            acc[fm][fn] = mfma_16x16x32_bf16(f.af[fm], f.bfr[fn], acc[fm][fn]);
          } else if constexpr (F == F_FP8) {
            const f32x4_t t = mfma_f8(f.af[fm], f.bfr[fn]);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[fm][fn][q] = __builtin_fmaf(t[q], f.as_[fm][q] * f.wsc[fn], acc[fm][fn][q]);
          } else {
            const i32x4_t v = f.bfr[fn];
            acc[fm][fn] = mfma_mx(f.af[fm], i32x8_t{v[0], v[1], v[2], v[3], 0, 0, 0, 0}, acc[fm][fn], f.sa[fm], f.sb[fn]);
          }
        }
      }
    };
    // Make step sn visible to every wave and refill the ring: this wave's
    // reads of the slot about to be refilled are done (lgkmcnt), its copies
    // of step sn have landed (vmcnt: D - 1 later steps may stay in flight),
    // then the barrier, then the copies of step sn + D into the slot of step
    // sn - 1.  Every step issues one step of copies (past the end: step
    // nk - 1 again, into slots no later step reads), so the wait count is
    // the same every time.
    auto next_step = [&](int sn) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), no other count
      wait_vm<(D - 1) * LS>();
      barrier_no_fence();
      issue(sn + D < nk ? sn + D : nk - 1, (sn + D) % NS);
    };

#pragma unroll
    for (int s = 0; s < D; ++s) issue(s < nk ? s : nk - 1, s % NS);
    if constexpr (F == F_BF16) {
      // Software pipeline: the fragments of the next sub-step are read from
      // LDS while the matrix cores work on the current one.
      // The last step is peeled so the loop body is straight-line code and
      // the LDS read counts the compiler waits for are exact; scheduling
      // barriers keep each group of reads ahead of the multiplies they
      // overlap with.
      Frag f0, f1;
      next_step(0);
      rd(0, 0, f0);
      for (int s = 0; s + 1 < nk; ++s) {
        rd(s, 1, f1);
        __builtin_amdgcn_sched_barrier(0);
        mm(f0);
        __builtin_amdgcn_sched_barrier(0);
        next_step(s + 1);
        rd(s + 1, 0, f0);
        __builtin_amdgcn_sched_barrier(0);
        mm(f1);
        __builtin_amdgcn_sched_barrier(0);
      }
      rd(nk - 1, 1, f1);
      mm(f0);
      mm(f1);
    } else {
      // one fragment buffer; a second does not fit the register file next
      // to the accumulators at BLOCK_M 128
      for (int s = 0; s < nk; ++s) {
        next_step(s);
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks) {
          Frag f0;
          rd(s, ks, f0);
          mm(f0);
        }
      }
    }
    wait_vm<0>();     // the copies past the last step have landed too
    __syncthreads();  // every wave is done reading the stage buffers

    // ---------------------------------------------------------------- epilogue
    if (G1) {
      constexpr int FA = FN / 2;
      constexpr int BNA = BNW / 2;
      float v[FM][FA][4];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fa = 0; fa < FA; ++fa)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[fm][fa][i] = swiglu(acc[fm][fa][i], acc[fm][fa + FA][i], p.lim);
      const int lcol0 = wn * (BNA / WN);  // first tile column of this wave
      if (F == F_BF16) {
        uint16_t* st = reinterpret_cast<uint16_t*>(lds);  // [BM][BNA]
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int fa = 0; fa < FA; ++fa)
              st[(wm * (BM / 2) + fm * 16 + 4 * g + i) * BNA + lcol0 + fa * 16 + r] =
                  (uint16_t)f32_to_bf16_bits(v[fm][fa][i]);
      } else if (F == F_FP8) {
        float* xch = reinterpret_cast<float*>(lds + BM * BNA);  // [WN][BM] after the byte tile
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float mm = 0.f;
#pragma unroll
            for (int fa = 0; fa < FA; ++fa) mm = fmaxf(mm, fabsf(v[fm][fa][i]));
            mm = row_max16(mm);  // the 16 lanes (one DPP row) of the row
            if (r == 0) xch[wn * BM + wm * (BM / 2) + fm * 16 + 4 * g + i] = mm;
          }
        __syncthreads();
        float* act_s = static_cast<float*>(p.act_s);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int lr = wm * (BM / 2) + fm * 16 + 4 * g + i;
            float amax = xch[lr];
#pragma unroll
            for (int w2 = 1; w2 < WN; ++w2) amax = fmaxf(amax, xch[w2 * BM + lr]);
            const float sc = fp8_group_scale(amax);
            if (wn == 0 && r == 0) act_s[(size_t)(blk * BM + lr) * (p.F / 128) + nt] = sc;
#pragma unroll
            for (int fa = 0; fa < FA; ++fa)
              lds[lr * BNA + lcol0 + fa * 16 + r] = (uint8_t)to_e4m3(fp8_scaled(v[fm][fa][i], sc));
          }
      } else {  // F_MX: groups of 32 columns = fragment pairs of this wave
        uint8_t* act_s = static_cast<uint8_t*>(p.act_s);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int lr = wm * (BM / 2) + fm * 16 + 4 * g + i;
#pragma unroll
            for (int gp = 0; gp < FA / 2; ++gp) {
              const float mm = row_max16(fmaxf(fabsf(v[fm][2 * gp][i]), fabsf(v[fm][2 * gp + 1][i])));
              const uint32_t c = mx_group_code(mm);
              const float inv = e8m0_inv(c);
              const int lc = lcol0 + gp * 32;
              if (r == 0) act_s[(size_t)(blk * BM + lr) * (p.F / 32) + (nt * BNA + lc) / 32] = (uint8_t)c;
              lds[lr * BNA + lc + r] = (uint8_t)to_e4m3(clamp448(v[fm][2 * gp][i] * inv));
              lds[lr * BNA + lc + 16 + r] = (uint8_t)to_e4m3(clamp448(v[fm][2 * gp + 1][i] * inv));
            }
          }
      }
      __syncthreads();
      // whole rows of the tile to act (BNA columns of 2 or 1 bytes)
      constexpr int RB = BNA * T::AB;  // bytes per tile row
      constexpr int CH = RB / 16;
      for (int idx = tid; idx < BM * CH; idx += NT) {
        const int lr = idx / CH;
        const int c = idx % CH;
        const uint4 val = *reinterpret_cast<const uint4*>(lds + lr * RB + c * 16);
        *reinterpret_cast<uint4*>(p.act + ((size_t)(blk * BM + lr) * p.F + nt * BNA) * T::AB + c * 16) = val;
      }
    } else {
      RowScatter<NT, BNW * 2 / 16, BM> rows;
      rows.load_slots(p, blk * BM, BM, tid);
      uint16_t* st = reinterpret_cast<uint16_t*>(lds);  // [BM][BNW]
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            st[(wm * (BM / 2) + fm * 16 + 4 * g + i) * BNW + wn * (BNW / WN) + fn * 16 + r] =
                (uint16_t)f32_to_bf16_bits(acc[fm][fn][i]);
      __syncthreads();
      rows.store(p, lds, nt * BNW, tid);
    }
    if (!dyn) break;
    __syncthreads();  // this tile (and the last index read) is done with LDS
    if (tid == 0) *reinterpret_cast<volatile int*>(lds) = wpx + atomicAdd(p.queue + xcd, 1);
    __syncthreads();
    j = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int*>(lds));
    __syncthreads();  // every wave has the index before the copies overwrite it
  }
  // the last workgroup to finish leaves the counters at zero for the next
  // launch (every workgroup has made its last take before it counts itself)
  if (dyn && tid == 0 && atomicAdd(p.queue + 8, 1) == (int)gridDim.x - 1) {
#pragma unroll
    for (int x = 0; x < 9; ++x) p.queue[x] = 0;
  }
}

// ---------------------------------------------------------------------------
// Paired tiled kernel (bf16, BLOCK_M = 64 or 128, prefill).  A tile is up to
// two consecutive blocks of one expert (2 BLOCK_M rows) x 256 weight rows:
// each weight byte copied to LDS feeds twice the rows of a BLOCK_M x 256
// tile, and the copy stream (what limits the tiled kernels: a CU keeps a
// fixed number of line requests in flight) carries fewer bytes per flop.
// Blocks pair up from the start of each expert's run (pair_table_kernel); an
// expert with an odd number of blocks ends in a single-block tile, whose
// missing half is neither copied (an empty buffer range returns zeros
// without touching memory) nor multiplied.  8 waves as 2 x 4, two per SIMD,
// each one block's rows x 64 weight rows (GEMM1: 32 gate rows and the
// matching 32 up rows); K steps of 128 bytes per row (two 32-wide MFMA
// steps) with separate LDS rings for A (two slots, one step ahead) and B
// (three slots, two steps ahead).  Per sub-step a wave reads its weight
// fragments, then its A fragments one at a time, each read issued before
// the MFMAs of the previous one.

// Pair table: tab[0] = number of pairs, tab[1 + j] = first block of pair j
// (bits 0-28), bit 30 set when the pair holds two blocks, and the window
// bits of pair_tile (common.h): bit 29 when pair j + 1 is the next pair of
// the same expert and j is an even pair of its expert, bit 31 when j is an
// odd one.  One workgroup walks the blocks 1024 at a time: an inclusive
// max-scan of the run starts gives each block the first block of its
// expert's run, a sum-scan numbers the blocks that start a pair (an even
// distance from that first block).
__global__ __launch_bounds__(1024) void pair_table_kernel(const int32_t* be, const int32_t* npp, int bm,
                                                          int32_t* tab) {
  __shared__ int s_max[16];
  __shared__ int s_cnt[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nblk = *npp / bm;
  int carry_first = 0;  // first block of the run that reaches the chunk's start
  int carry_pairs = 0;
  for (int c0 = 0; c0 < nblk; c0 += 1024) {
    const int b = c0 + tid;
    const bool valid = b < nblk;
    const int e = valid ? be[b] : -1;
    const bool first = valid && (b == 0 || be[b - 1] != e);
    int m = first ? b : -1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(m, off, 64);
      if (lane >= off) m = max(m, o);
    }
    if (lane == 63) s_max[wave] = m;
    __syncthreads();
    for (int w = 0; w < wave; ++w) m = max(m, s_max[w]);
    const int fb = max(m, carry_first);
    const bool start = valid && ((b - fb) & 1) == 0;
    const uint64_t bal = __ballot(start);
    const int pos = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0, cf = carry_first;
    for (int w = 0; w < 16; ++w) {
      const int c = s_cnt[w];
      before += w < wave ? c : 0;
      total += c;
      cf = max(cf, s_max[w]);
    }
    if (start) {
      const bool two = b + 1 < nblk && be[b + 1] == e;
      const bool next = b + 2 < nblk && be[b + 2] == e;  // the expert has another pair
      const bool odd = ((b - fb) >> 1) & 1;              // pair index within the expert
      tab[1 + carry_pairs + before + pos] = pair_entry(b, two, !odd && next, odd);
    }
    carry_first = cf;
    carry_pairs += total;
    __syncthreads();  // s_max / s_cnt are rewritten by the next chunk
  }
  if (tid == 0) tab[0] = carry_pairs;
}

template <bool G1, int NW, int BB>  // BB: rows per block (64 or 128)
__global__ __launch_bounds__(64 * NW) void gemm_pair_bf16(GemmP p) {
  constexpr int BMT = 2 * BB;     // rows per tile
  constexpr int BNW = 256;        // weight rows per tile
  constexpr int NT = 64 * NW;
  constexpr int WN = NW / 2;      // waves: 2 along M x WN along N
  // K steps of 128 bytes per row (two 32-wide MFMA steps): every copy
  // request is a whole 128-byte line (a CU keeps a fixed number of requests
  // in flight, so the request size sets its copy rate).  A and B have rings
  // of their own: A two 32 KiB slots, one step ahead; B (the weights, whose
  // reads go to HBM) three slots, two steps ahead.
  constexpr int RB = 128;
  constexpr int CPR = RB / 16;    // 16-byte chunks per row and step
  constexpr int KS = RB / 64;     // MFMA steps per K step
  constexpr int ASZ = BMT * RB;
  constexpr int BSZ = BNW * RB;
  constexpr int NA = 2, NB = 3;
  constexpr int DA = NA - 1, DB = NB - 1;  // steps each ring runs ahead
  constexpr int FM = BB / 16;        // 16-row fragments per wave (one block's rows)
  constexpr int FN = BNW / WN / 16;  // 16-column fragments per wave
  constexpr int RW = BMT / NW;       // A rows each wave copies
  constexpr int RWB = BNW / NW;      // weight rows each wave copies
  constexpr int LA = BMT * CPR / NT;  // copy instructions per wave per step (1 KiB each)
  constexpr int LB = BNW * CPR / NT;
  constexpr int LS = LA + LB;
  static_assert(LB <= 63 && (!G1 || FN % 2 == 0) && NA * ASZ + NB * BSZ <= 163840, "rings / vmcnt / gate-up pairs");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave / WN;  // rows [BB wm, +BB): the tile's first or second block
  const int wn = wave % WN;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int K = G1 ? p.H : p.F;
  const int N = G1 ? p.F : p.H;
  const int BNO = G1 ? BNW / 2 : BNW;  // output columns per tile
  const int ntn = N / BNO;
  const int nblk = *p.npp / BB;
  // a pair table left by another shape holds more pairs than blocks exist:
  // at most one pair per block, and tiles past the blocks are skipped
  const int npairs = min(p.pairs[0], nblk);
  const int64_t n_valid = (int64_t)npairs * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int nk = K / (RB / 2);
  const int rowbytes = K * 2;
  const uint8_t* asrc = G1 ? p.x : p.act;
  const uint8_t* wsrc = G1 ? p.w13 : p.w2;
  const size_t erows = G1 ? (size_t)2 * p.F : (size_t)p.H;
  const rsrc_t ra = make_rsrc(asrc, (uint64_t)(G1 ? p.A / p.k : nblk * BB) * rowbytes);
  const rsrc_t rnone = make_rsrc(asrc, 0);  // every read returns zero

  // LDS layout of a slot: 128-byte rows, 16-byte chunk c of row rr at slot
  // c ^ (rr / 2 % 8), as in gemm_tiled: a fragment read (16 rows x 4
  // chunks) then hits no bank twice
  auto lds_off = [](int rr, int c) { return rr * RB + 16 * (c ^ ((rr >> 1) & (CPR - 1))); };
  // the tile row and chunk whose bytes copy lane `lane` of an instruction
  // that fills 64 / CPR rows from row0 on (1 KiB, lane l at byte 16 l)
  auto copy_src = [](int row0, int lane, int& rr, int& c) {
    rr = row0 + lane / CPR;
    c = (lane % CPR) ^ ((rr >> 1) & (CPR - 1));
  };
  // GEMM1: the first FN / 2 fragments are gate rows, the rest the matching up rows
  auto frag_lrow = [&](int fn) {
    return G1 ? (fn < FN / 2 ? wn * (BNW / (2 * WN)) + fn * 16 : BNW / 2 + wn * (BNW / (2 * WN)) + (fn - FN / 2) * 16)
              : wn * (BNW / WN) + fn * 16;
  };
  auto weight_row = [&](int nt, int lrow) {
    if (G1) return lrow < BNW / 2 ? nt * (BNW / 2) + lrow : p.F + nt * (BNW / 2) + (lrow - BNW / 2);
    return nt * BNW + lrow;
  };

  // Tiles: XCD x (workgroups are dealt to the XCDs round-robin) owns the
  // contiguous run [x per, x per + per) of logical tiles.  A workgroup's
  // first tile is its index among the XCD's workgroups; when the XCD has
  // more tiles than workgroups, each takes the next one from the XCD's
  // counter when it is done with the last, so the CUs of an XCD end within
  // one tile of each other.  The index goes through the first LDS word
  // while the ring is idle.
  const int xcd = blockIdx.x & 7;
  const int wpx = (int)(gridDim.x >> 3);  // workgroups per XCD
  const bool dyn = per > wpx;
  int j = (int)(blockIdx.x >> 3);
  for (;; ) {
    const int64_t L = (int64_t)xcd * per + j;
    if (j >= per || L >= n_valid) break;
    // tile values are uniform; readfirstlane keeps them (and the buffer
    // descriptors made from them) in scalar registers
    // plain pair-major order (measured: interleaving an expert's pairs left
    // the MXFP4 kernel 1-3 % faster and this one's GEMM1 2 % slower at
    // Qwen3 T=4096)
    const PairTile pt = pair_tile<false>(p.pairs, npairs, L, ntn);
    const int nt = pt.nt;
    const int blk = pt.blk;  // first block of the tile
    const bool two = pt.two;
    if (blk + (two ? 1 : 0) < nblk) {
      const int e = __builtin_amdgcn_readfirstlane(p.block_expert[blk]);
      const bool mine = wm == 0 || two;  // this wave's block exists

      // wave w copies tile rows [RW w, RW w + RW): rows of the second block
      // come from an empty range when the tile holds one block
      const bool copy_rows = wave < NW / 2 || two;
      const rsrc_t rA = copy_rows ? ra : rnone;
      uint32_t ag[LA];
  #pragma unroll
      for (int i = 0; i < LA; ++i) {
        int row, c;
        copy_src(wave * RW + (64 / CPR) * i, lane, row, c);
        bool v;
        const int src = copy_rows ? a_row_index<G1>(p, blk, BB, row, v) : 0;  // padding rows read token 0
        ag[i] = (uint32_t)src * rowbytes + 16 * c;
      }
      const rsrc_t rb = make_rsrc(wsrc + (size_t)e * erows * rowbytes, (uint64_t)erows * rowbytes);
      uint32_t bg[LB];
  #pragma unroll
      for (int i = 0; i < LB; ++i) {
        int row, c;
        copy_src(wave * RWB + (64 / CPR) * i, lane, row, c);
        bg[i] = (uint32_t)weight_row(nt, row) * rowbytes + 16 * c;
      }
      // copies of step s (clamped to the last step: past the end a step is
      // copied again into a slot no later step reads, so every barrier waits
      // for the same count)
      auto issue_a = [&](int s) {
        uint8_t* st = lds + (s % NA) * ASZ;
        s = s < nk ? s : nk - 1;
  #pragma unroll
        for (int i = 0; i < LA; ++i) buf2lds16(rA, ag[i], s * RB, st + (wave * RW + (64 / CPR) * i) * RB);
      };
      auto issue_b = [&](int s) {
        uint8_t* st = lds + NA * ASZ + (s % NB) * BSZ;
        s = s < nk ? s : nk - 1;
  #pragma unroll
        for (int i = 0; i < LB; ++i) buf2lds16(rb, bg[i], s * RB, st + (wave * RWB + (64 / CPR) * i) * RB);
      };

      f32x4_t acc[FM][FN];
  #pragma unroll
      for (int fm = 0; fm < FM; ++fm)
  #pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // Before step sn: this wave's LDS reads are done (lgkmcnt), its copies
      // of A(sn) and B(sn) have landed (vmcnt: only B(sn + 1), the copies
      // issued last, may remain), barrier, then A(sn + 1) into the A slot of
      // step sn - 1 and B(sn + 2) into the B slot of step sn - 1.
      auto next_step = [&](int sn) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), no other count
        wait_vm<LB>();
        barrier_no_fence();
        issue_a(sn + DA);
        issue_b(sn + DB);
      };

      issue_a(0);
      issue_b(0);
      issue_b(1);
      for (int s = 0; s < nk; ++s) {
        next_step(s);
        if (mine) {
          // per 32-wide sub-step: the weight fragments, then the A fragments
          // one at a time, each read issued before the MFMAs of the previous
          // (measured, Qwen3 T=4096: GEMM1 344 -> 330 us against reading all
          // fragments of a sub-step, then multiplying)
          const uint8_t* As = lds + (s % NA) * ASZ;
          const uint8_t* Bs = lds + NA * ASZ + (s % NB) * BSZ;
  #pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            bf16x8_t bfr[FN];
  #pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              bfr[fn] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(frag_lrow(fn) + r, 4 * ks + g));
            auto read_a = [&](int fm) {
              return *reinterpret_cast<const bf16x8_t*>(As + lds_off(wm * BB + fm * 16 + r, 4 * ks + g));
            };
            auto mult = [&](int fm, const bf16x8_t& a) {
  #pragma unroll
              for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32_bf16(a, bfr[fn], acc[fm][fn]);
            };
            bf16x8_t a0 = read_a(0), a1;
  #pragma unroll
            for (int fm = 0; fm < FM; fm += 2) {
              a1 = read_a(fm + 1);
              __builtin_amdgcn_sched_barrier(0);
              mult(fm, a0);
              __builtin_amdgcn_sched_barrier(0);
              if (fm + 2 < FM) a0 = read_a(fm + 2);
              __builtin_amdgcn_sched_barrier(0);
              mult(fm + 1, a1);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      wait_vm<0>();     // the copies past the last step have landed too
      __syncthreads();  // every wave is done reading the rings

      // ---------------------------------------------------------------- epilogue
      const int nrows = two ? BMT : BB;
      if (G1) {
        constexpr int BNA = BNW / 2;  // SwiGLU columns per tile
        uint16_t* st = reinterpret_cast<uint16_t*>(lds);  // [BMT][BNA]
  #pragma unroll
        for (int fm = 0; fm < FM; ++fm)
  #pragma unroll
          for (int i = 0; i < 4; ++i)
  #pragma unroll
            for (int fa = 0; fa < FN / 2; ++fa)
              st[(wm * BB + fm * 16 + 4 * g + i) * BNA + wn * (BNA / WN) + fa * 16 + r] =
                  (uint16_t)f32_to_bf16_bits(swiglu(acc[fm][fa][i], acc[fm][fa + FN / 2][i], p.lim));
        __syncthreads();
        constexpr int CH = BNA * 2 / 16;  // 16-byte chunks per tile row
        for (int idx = tid; idx < nrows * CH; idx += NT) {
          const int lr = idx / CH;
          const int c = idx % CH;
          const uint4 val = *reinterpret_cast<const uint4*>(lds + lr * BNA * 2 + c * 16);
          *reinterpret_cast<uint4*>(p.act + ((size_t)(blk * BB + lr) * p.F + nt * BNA) * 2 + c * 16) = val;
        }
      } else {
        RowScatter<NT, BNW * 2 / 16, BMT> rows;
        rows.load_slots(p, blk * BB, nrows, tid);
        uint16_t* st = reinterpret_cast<uint16_t*>(lds);  // [BMT][BNW]
  #pragma unroll
        for (int fm = 0; fm < FM; ++fm)
  #pragma unroll
          for (int i = 0; i < 4; ++i)
  #pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              st[(wm * BB + fm * 16 + 4 * g + i) * BNW + wn * (BNW / WN) + fn * 16 + r] =
                  (uint16_t)f32_to_bf16_bits(acc[fm][fn][i]);
        __syncthreads();
        rows.store(p, lds, nt * BNW, tid);
      }
    }
    if (!dyn) break;
    __syncthreads();  // this tile (and the last index read) is done with LDS
    if (tid == 0) *reinterpret_cast<volatile int*>(lds) = wpx + atomicAdd(p.queue + xcd, 1);
    __syncthreads();
    j = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int*>(lds));
    __syncthreads();  // every wave has the index before the copies overwrite it
  }
  // the last workgroup to finish leaves the counters at zero for the next
  // launch (every workgroup has made its last take before it counts itself)
  if (dyn && tid == 0 && atomicAdd(p.queue + 8, 1) == (int)gridDim.x - 1) {
#pragma unroll
    for (int x = 0; x < 9; ++x) p.queue[x] = 0;
  }
}

// ---------------------------------------------------------------------------
// Paired tiled kernel for MXFP4 weights (BLOCK_M = 64 or 128, prefill): the
// tile of gemm_pair_bf16 (up to two consecutive blocks of one expert x 256
// weight rows; 8 waves as 2 x 4, each one block's rows x 64 weight rows) on
// e4m3 activations x e2m1 weights.  Each weight tile is copied once for
// both blocks.  A K step is one 128-wide MFMA step: 128 bytes of each A row
// and 64 bytes of each weight row.
//
// Copies.  Waves 0-3 copy the A rows (one step ahead: they come from the L2,
// where the rows of a pair serve all its N tiles) and waves 4-7 the weight
// rows (three steps ahead: they come from HBM).  A wave's copies complete in
// issue order, so a wave that copied both would have to wait for its
// younger weight copies whenever it waits for an A step; split, each half
// waits for its own stream only.  LDS: two A slots, four weight slots and
// two slots of e8m0 scales, 144 KiB at BB = 128 (four steps ahead in five
// slots, 160 KiB, took 2-3 % longer in both GEMMs, DSV4 T=8192; two ahead
// longer again).  The scales (one byte per row and 32-wide K group) are
// copied 16 bytes per row at a time, four steps' worth (a CU keeps a fixed
// number of copy requests in flight).
//
// Tiles.  Each workgroup loops over tiles from its XCD's queue.  GEMM1
// issues the next tile's copies ahead of step 0 before its epilogue, which
// then runs while they land; the weight waves store the epilogue's rows.
//
// Multiply.  Per step a wave reads its weight fragments, then its A
// fragments one at a time, each read issued before the MFMAs of the
// previous one so that LDS latency overlaps the matrix cores.  GEMM1's
// epilogue requantises each row's 32 SwiGLU columns of a wave (one MX group)
// with the power-of-two scale pow2_at_least(amax / 448) ([MegaMoE] §3.5).
// Ring depth of the paired MXFP4 kernels: A slots (the A stream copies
// MOE_MX_A_SLOTS - 1 steps ahead) and weight slots (MOE_MX_B_SLOTS - 1 ahead).
#ifndef MOE_MX_A_SLOTS
#define MOE_MX_A_SLOTS 2
#endif
#ifndef MOE_MX_B_SLOTS
#define MOE_MX_B_SLOTS 4
#endif
template <bool G1, int BB>  // BB: rows per block (64 or 128)
__global__ __launch_bounds__(512) void gemm_pair_mx(GemmP p) {
  constexpr int NW = 8, NT = 64 * NW, WN = NW / 2;
  constexpr int BMT = 2 * BB;          // rows per tile
  constexpr int BNW = 256;             // weight rows per tile
  constexpr int ARB = 128, BRB = 64;   // A / B bytes per row and step
  constexpr int ASZ = BMT * ARB;       // one A slot
  constexpr int BSZ = BNW * BRB;       // one weight slot
  constexpr int NA = MOE_MX_A_SLOTS, NB = MOE_MX_B_SLOTS;  // ring slots (A, weights)
  constexpr int DA = NA - 1, DB = NB - 1;                    // steps copied ahead
  constexpr int SCG = 4;               // steps per scale group
  constexpr int SCSZ = NT * 16;        // a scale group: 16 bytes per row, A rows then weight rows
  constexpr int FM = BB / 16;          // 16-row fragments per wave (one block's rows)
  constexpr int FN = BNW / WN / 16;    // 16-column fragments per wave
  constexpr int CW = NW / 2;           // waves per copy stream
  constexpr int RA = BMT / CW;         // A rows each A wave copies
  constexpr int RB = BNW / CW;         // weight rows each weight wave copies
  constexpr int LA = RA / 8;           // 1 KiB copies per step: 8 A rows of 128 bytes
  constexpr int LB = RB / 16;          //                        16 weight rows of 64 bytes
  constexpr int ABASE = 0, BBASE = NA * ASZ, SBASE = NA * ASZ + NB * BSZ;
  // most stores per weight wave that a GEMM1 epilogue issues after the next
  // tile's first copies (rows of BNW / 2 bytes in 16-byte pieces over 256
  // threads); GEMM2 stores before them
  constexpr int SXM = G1 ? BMT * (BNW / 32) / (NT / 2) : 0;
  static_assert(BMT <= CW * 64 && BNW == CW * 64 && SBASE + 2 * SCSZ <= 163840 && LA >= 1 && LB >= 1 &&
                FN % 2 == 0 && LB * (DB - 1) + DB + SXM <= 63 && LA * (DA - 1) + DA + SXM <= 63 && FM % 2 == 0 &&
                DA >= 1 && DB >= 1, "tile, LDS, copies and vmcnt");
  // a scale group goes out after the copies of the step D before its first
  // step; with D < SCG that is before the copies of its first step
  static_assert(DA < SCG && DB < SCG, "scale groups land before the steps that read them");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool bwave = wave >= CW;  // copies weight rows (else A rows)
  const int bt = tid - CW * 64;   // weight waves: thread index among them
  const int cw = wave % CW;       // index among the waves of its copy stream
  const int lane = tid & 63;
  const int wm = wave / WN;  // rows [BB wm, +BB): the tile's first or second block
  const int wn = wave % WN;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int K = G1 ? p.H : p.F;
  const int N = G1 ? p.F : p.H;
  const int BNO = G1 ? BNW / 2 : BNW;  // output columns per tile
  const int ntn = N / BNO;
  const int nblk = *p.npp / BB;
  // a pair table left by another shape holds more pairs than blocks exist:
  // at most one pair per block, and tiles past the blocks are skipped
  const int npairs = min(p.pairs[0], nblk);
  const int64_t n_valid = (int64_t)npairs * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int nk = K / 128;              // a multiple of SCG (K is a multiple of 512)
  const int ng = nk / SCG;
  const int rowbytes_a = K;       // e4m3
  const int rowbytes_b = K / 2;   // packed e2m1
  const int kgroups = K / 32;     // e8m0 scale bytes per row
  const uint8_t* asrc = G1 ? p.x : p.act;
  const uint8_t* wsrc = G1 ? p.w13 : p.w2;
  const uint8_t* ascale = static_cast<const uint8_t*>(G1 ? p.xs : p.act_s);
  const uint8_t* wscale = static_cast<const uint8_t*>(G1 ? p.w13_s : p.w2_s);
  const size_t erows = G1 ? (size_t)2 * p.F : (size_t)p.H;
  const uint32_t arows = G1 ? (uint32_t)(p.A / p.k) : (uint32_t)nblk * BB;
  const rsrc_t ra = make_rsrc(asrc, (uint64_t)arows * rowbytes_a);
  const rsrc_t rnone = make_rsrc(asrc, 0);  // every read returns zero
  const rsrc_t ras = make_rsrc(ascale, (uint64_t)arows * kgroups);

  // LDS chunk slots: A rows of 128 bytes, chunk c at c ^ (rr / 2 % 8);
  // weight rows of 64 bytes, chunk c at c ^ (rr / 2 % 4) (a fragment read of
  // 16 rows then hits no bank twice)
  auto a_off = [](int rr, int c) { return rr * ARB + 16 * (c ^ ((rr >> 1) & 7)); };
  auto b_off = [](int rr, int c) { return rr * BRB + 16 * (c ^ ((rr >> 1) & 3)); };
  // GEMM1: the first FN / 2 fragments are gate rows, the rest the matching up rows
  auto frag_lrow = [&](int fn) {
    return G1 ? (fn < FN / 2 ? wn * (BNW / (2 * WN)) + fn * 16 : BNW / 2 + wn * (BNW / (2 * WN)) + (fn - FN / 2) * 16)
              : wn * (BNW / WN) + fn * 16;
  };
  auto weight_row = [&](int nt, int lrow) {
    if (G1) return lrow < BNW / 2 ? nt * (BNW / 2) + lrow : p.F + nt * (BNW / 2) + (lrow - BNW / 2);
    return nt * BNW + lrow;
  };

  // Tiles as gemm_pair_bf16: XCD x owns the contiguous run [x per, +per) of
  // logical (pair-major) tiles, first tiles by index, then per-XCD queues.
  const int xcd = blockIdx.x & 7;
  const int wpx = (int)(gridDim.x >> 3);
  const bool dyn = per > wpx;
  auto in_range = [&](int jx) { return jx < per && (int64_t)xcd * per + jx < n_valid; };

  // One tile's copy state: its blocks and N tile, and the copy sources of
  // this wave's stream.  Only GEMM1's A rows are gathered (cg, per tile); the
  // other streams read rows at a fixed offset from the tile's first one: a
  // per-lane offset set once (cl) plus the tile's wave-uniform byte offset so,
  // which rides in the copy's scalar offset.
  constexpr int LC = LA > LB ? LA : LB;
  struct Tile {
    int nt, blk, e;
    bool two;
    bool ok;         // the tile lies inside the blocks (tiles of a stale pair table are skipped)
    bool copy_rows;  // A waves: this wave's rows exist
    uint32_t sg;
    uint32_t so;
    uint32_t cg[G1 ? LC : 1];
  };
  uint32_t cl[LC];
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    if (bwave) {
      const int rr = cw * RB + 16 * i + lane / 4;
      const int c = (lane % 4) ^ ((rr >> 1) & 3);
      cl[i] = i < LB ? (uint32_t)weight_row(0, rr) * rowbytes_b + 16 * c : 0u;
    } else {
      const int rr = cw * RA + 8 * i + lane / 8;
      const int c = (lane % 8) ^ ((rr >> 1) & 7);
      cl[i] = (G1 ? 0u : (uint32_t)rr * rowbytes_a) + 16 * c;
    }
  }
  // the copy sources as buffer descriptors (rebuilt from the tile's fields:
  // kept in a struct, the descriptor type ended up in scratch memory)
  auto src_rc = [&](const Tile& t) {
    return bwave ? make_rsrc(wsrc + (size_t)t.e * erows * rowbytes_b, (uint64_t)erows * rowbytes_b)
                 : (t.copy_rows ? ra : rnone);
  };
  auto src_rs = [&](const Tile& t) {
    return bwave ? make_rsrc(wscale + (size_t)t.e * erows * kgroups, (uint64_t)erows * kgroups) : ras;
  };
  auto setup = [&](int jx) {
    Tile t;
    // an expert's pairs interleaved by N tile (measured, DSV4 T=8192: GEMM1
    // 1155 -> 1140 us, GEMM2 598 -> 581 us)
    const PairTile pt = pair_tile<true>(p.pairs, npairs, (int64_t)xcd * per + jx, ntn);
    t.nt = pt.nt;
    t.blk = pt.blk;
    t.two = pt.two;
    t.ok = pt.blk + (pt.two ? 1 : 0) < nblk;
    t.e = 0;
    t.copy_rows = false;
    t.sg = 0u;
    t.so = 0u;
#pragma unroll
    for (int i = 0; i < (G1 ? LC : 1); ++i) t.cg[i] = 0u;
    if (!t.ok) return t;
    t.e = __builtin_amdgcn_readfirstlane(p.block_expert[t.blk]);
    // This wave's copy stream.  A waves: tile rows [RA cw, +RA), 8 per
    // instruction (rows of a missing second block from the empty range).
    // Weight waves: weight rows [RB cw, +RB), 16 per instruction.
    t.copy_rows = (cw * RA < BB) || t.two;
    if (bwave) t.so = (uint32_t)(t.nt * BNO) * rowbytes_b;
    else if (!G1) t.so = (uint32_t)(t.blk * BB) * rowbytes_a;  // GEMM2's A rows are the padded rows themselves
    if constexpr (G1) {
      if (!bwave) {
#pragma unroll
        for (int i = 0; i < LC; ++i) {
          const int rr = cw * RA + 8 * i + lane / 8;
          bool v;
          const int src = (i < LA && t.copy_rows) ? a_row_index<G1>(p, t.blk, BB, rr, v) : 0;  // padding: row 0
          t.cg[i] = (uint32_t)src * rowbytes_a + cl[i];
        }
      }
    }
    // scale groups: 16 bytes of A row q (A waves, q = tid < BMT; the rest
    // and rows of a missing block read the tile's first row) or of weight
    // row q = tid - 256 (weight waves); the descriptor is wave-uniform
    if (bwave) {
      t.sg = (uint32_t)weight_row(t.nt, tid - CW * 64) * kgroups;
    } else {
      const int q = tid < BMT ? tid : 0;
      bool v;
      t.sg = (uint32_t)a_row_index<G1>(p, t.blk, BB, (q < BB || t.two) ? q : 0, v) * kgroups;
    }
    return t;
  };
  // step s's copies of this wave's stream (none past the last step)
  auto issue = [&](const Tile& t, int s) {
    if (s >= nk) return;
    const rsrc_t rc = src_rc(t);
    if (bwave) {
      uint8_t* st = lds + BBASE + (s % NB) * BSZ + cw * RB * BRB;
#pragma unroll
      for (int i = 0; i < LB; ++i) buf2lds16(rc, cl[i], t.so + s * BRB, st + 16 * i * BRB);
    } else {
      uint8_t* st = lds + ABASE + (s % NA) * ASZ + cw * RA * ARB;
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        if constexpr (G1) buf2lds16(rc, t.cg[i], s * ARB, st + 8 * i * ARB);
        else buf2lds16(rc, cl[i], t.so + s * ARB, st + 8 * i * ARB);
      }
    }
  };
  auto issue_sc = [&](const Tile& t, int G) {
    if (G >= ng) return;
    buf2lds16(src_rs(t), t.sg, G * 16, lds + SBASE + (G & 1) * SCSZ + wave * 1024);
  };
  // the copies ahead of step 0: scale group 0, then A steps 0 .. DA - 1 or
  // weight steps 0 .. DB - 1 (into the first DA / DB slots, scale slot 0)
  auto prologue = [&](const Tile& t) {
    issue_sc(t, 0);
    if (bwave) {
#pragma unroll
      for (int s = 0; s < DB; ++s) issue(t, s);
    } else {
#pragma unroll
      for (int s = 0; s < DA; ++s) issue(t, s);
    }
  };


  // Taking a tile from the XCD's queue: thread 0's atomic, then the index
  // through an LDS word (in scale slot 1, which the copies ahead of a tile's
  // step 0 leave alone) and one barrier.
  int* const ctl = reinterpret_cast<int*>(lds + SBASE + SCSZ);
  int taken = 0;
  auto take_issue = [&]() {
    if (tid == 0) taken = atomicAdd(p.queue + xcd, 1);
  };
  // (the word is accessed as LDS: through a generic pointer it would take
  // flat instructions, whose waits cover every vector memory operation)
  volatile lds_int_t* const ctl3 = (volatile lds_int_t*)ctl;
  auto take_finish = [&]() {
    if (tid == 0) *ctl3 = wpx + taken;
    lds_barrier();
    return __builtin_amdgcn_readfirstlane(*ctl3);
  };

  f32x4_t acc[FM][FN];
  int j = (int)(blockIdx.x >> 3);
  if (in_range(j)) {
    // GEMM1 (PF) issues the next tile's copies ahead of step 0 before its
    // epilogue, so they land while the SwiGLU and requantisation run; the
    // queue is read one tile ahead for that.  (GEMM2 staging its output in
    // quarters to do the same measured slower, DSV4 T=8192: 572 -> 724 us.)
    constexpr bool PF = G1;
    Tile cur = setup(j);
    int jn = per;  // the next tile (per: none)
    if (dyn) {
      take_issue();
      jn = take_finish();
    }
    bool pre = false;  // cur's copies ahead of step 0 are in flight
    // stores this wave issued after cur's copies ahead of step 0 (a lower
    // bound): the waits of steps 0 .. D - 1 leave them in flight too
    // (vector memory operations complete in issue order)
    int sx = 0;
    for (;;) {
      const bool mine = wm == 0 || cur.two;  // this wave's block exists
      if (cur.ok) {
        if (!pre) {
          prologue(cur);
          sx = 0;
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < nk; ++s) {
          // Every wave has read the slots about to be refilled (lgkmcnt(0))
          // and this wave's copies of step s have landed (the copies issued
          // after them stay in flight: copies_after).  Then the barrier, and
          // the copies of steps s + DA (A) / s + DB (weights) and of the
          // next scale group.
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), no other count
          const int sxs = s < (bwave ? DB : DA) ? sx : 0;
          if (bwave) wait_vm_upto<LB * (DB - 1) + DB + SXM>(copies_after<LB, DB, SCG>(s, nk, ng) + sxs);
          else wait_vm_upto<LA * (DA - 1) + DA + SXM>(copies_after<LA, DA, SCG>(s, nk, ng) + sxs);
          barrier_no_fence();
          issue(cur, s + (bwave ? DB : DA));
          if (s % SCG == 0) issue_sc(cur, s / SCG + 1);
          if (mine) {
            const uint8_t* As = lds + ABASE + (s % NA) * ASZ;
            const uint8_t* Bs = lds + BBASE + (s % NB) * BSZ;
            // row q's byte for K group g of step s: 16 q + 4 (s % 4) + g
            const uint8_t* Ss = lds + SBASE + ((s / SCG) & 1) * SCSZ + 4 * (s % SCG);
            i32x4_t bfr[FN];
            int sb[FN];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
              const int rr = frag_lrow(fn) + r;
              bfr[fn] = *reinterpret_cast<const i32x4_t*>(Bs + b_off(rr, g));
              sb[fn] = (int)Ss[(CW * 64 + rr) * 16 + g];
            }
            auto read_a = [&](int fm, i32x4_t& lo, i32x4_t& hi, int& sa) {
              const int rr = wm * BB + fm * 16 + r;
              lo = *reinterpret_cast<const i32x4_t*>(As + a_off(rr, g));
              hi = *reinterpret_cast<const i32x4_t*>(As + a_off(rr, 4 + g));
              sa = (int)Ss[rr * 16 + g];
            };
            auto mult = [&](int fm, const i32x4_t& lo, const i32x4_t& hi, int sa) {
              const i32x8_t af = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
              for (int fn = 0; fn < FN; ++fn) {
                const i32x4_t v = bfr[fn];
                acc[fm][fn] = mfma_mx(af, i32x8_t{v[0], v[1], v[2], v[3], 0, 0, 0, 0}, acc[fm][fn], sa, sb[fn]);
              }
            };
            // A fragments in two register sets: the reads of fragment fm + 1
            // go out before the MFMAs of fragment fm
            i32x4_t lo0, hi0, lo1, hi1;
            int sa0, sa1;
            read_a(0, lo0, hi0, sa0);
#pragma unroll
            for (int fm = 0; fm < FM; fm += 2) {
              read_a(fm + 1, lo1, hi1, sa1);
              __builtin_amdgcn_sched_barrier(0);
              mult(fm, lo0, hi0, sa0);
              __builtin_amdgcn_sched_barrier(0);
              if (fm + 2 < FM) read_a(fm + 2, lo0, hi0, sa0);
              __builtin_amdgcn_sched_barrier(0);
              mult(fm + 1, lo1, hi1, sa1);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        wait_vm<0>();     // the copies past the last step have landed too
        __syncthreads();  // every wave is done reading the rings
      } else {
        __syncthreads();  // every wave has read the last index (ctl is written again below)
      }

      const bool more = in_range(jn);
      Tile nx = cur;
      if (more) {
        take_issue();  // the tile after next, or past the end
        if (PF) {
          nx = setup(jn);
          if (nx.ok) prologue(nx);
        }
      }

      // ---------------------------------------------------------------- epilogue
      const int nrows = cur.two ? BMT : BB;
      constexpr int BNA = BNW / 2;  // GEMM1: SwiGLU columns per tile
      // GEMM1 stages its bytes in A slot NA - 1 and its codes in weight slot
      // NB - 1, which the copies ahead of the next tile's step 0 leave alone
      uint8_t* const stg = lds + ABASE + (NA - 1) * ASZ;
      uint8_t* const cds = lds + BBASE + (NB - 1) * BSZ;
      static_assert(BMT * BNA <= ASZ && BMT * (BNA / 32) <= BSZ && DB <= NB - 1, "epilogue staging");
      static_assert(G1 || BMT * BNW * 2 <= SBASE + SCSZ, "GEMM2's staged tile ends below the queue word");
      RowScatter<NT, BNW * 2 / 16, BMT> rows;
      if (cur.ok) {
        if (G1) {
          // this lane's first row (fm = 0, i = 0) in the byte tile and in the
          // code table; the others are compile-time offsets from it
          uint8_t* const rowp = stg + (wm * BB + 4 * g) * BNA + wn * 32 + r;
          uint8_t* const codep = cds + (wm * BB + 4 * g) * (BNA / 32) + wn;
          // the same code with and without the SwiGLU clamp (no limit: the
          // clamp's three instructions per value are left out)
          auto requant = [&](auto clamped) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float v0 = decltype(clamped)::value ? swiglu(acc[fm][0][i], acc[fm][FN / 2][i], p.lim)
                                                          : silu_mul(acc[fm][0][i], acc[fm][FN / 2][i]);
                const float v1 = decltype(clamped)::value ? swiglu(acc[fm][1][i], acc[fm][FN / 2 + 1][i], p.lim)
                                                          : silu_mul(acc[fm][1][i], acc[fm][FN / 2 + 1][i]);
                // the wave's 32 columns of row lr are one MX group: its amax
                // over the 16 lanes (one DPP row) that hold the row
                const float m = row_max16(fmaxf(fabsf(v0), fabsf(v1)));
                const uint32_t code = mx_group_code(m);
                const float inv = e8m0_inv(code);
                if (r == 0) codep[(fm * 16 + i) * (BNA / 32)] = (uint8_t)code;
                // |v| <= m <= 448 x scale for finite values: no clamp needed
                rowp[(fm * 16 + i) * BNA] = (uint8_t)to_e4m3(v0 * inv);
                rowp[(fm * 16 + i) * BNA + 16] = (uint8_t)to_e4m3(v1 * inv);
              }
          };
          if (p.lim < __builtin_inff()) requant(BoolTag<true>{});
          else requant(BoolTag<false>{});
        } else {
          rows.load_slots(p, cur.blk * BB, nrows, tid);
          uint16_t* st = reinterpret_cast<uint16_t*>(lds);  // [BMT][BNW]
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int fn = 0; fn < FN; ++fn)
                st[(wm * BB + fm * 16 + 4 * g + i) * BNW + wn * (BNW / WN) + fn * 16 + r] =
                    (uint16_t)f32_to_bf16_bits(acc[fm][fn][i]);
        }
      }
      // the staged tile is complete (and the next index is in ctl)
      sx = 0;
      int jnn = per;
      if (more) jnn = take_finish();
      else lds_barrier();
      if (cur.ok) {
        if (G1) {
          // the weight waves store (the A waves' first copies of the next
          // tile then wait for no store)
          uint8_t* acts = static_cast<uint8_t*>(p.act_s);
          if (bwave) {
            // the tile's BNA / 32 codes of a row are one 4-byte word of act_s
            if (bt < nrows)
              *reinterpret_cast<uint32_t*>(acts + (size_t)(cur.blk * BB + bt) * (p.F / 32) + cur.nt * (BNA / 32)) =
                  *reinterpret_cast<const uint32_t*>(cds + bt * (BNA / 32));
            // piece bt + it NT / 2 (it = 0 .. nrows / RPI - 1) of the tile:
            // chunk bt % CH of row bt / CH + it RPI, read two at a time
            constexpr int CH = BNA / 16;       // 16-byte chunks per tile row
            constexpr int RPI = NT / 2 / CH;   // rows per piece index step
            static_assert(NT / 2 % CH == 0 && BB % (2 * RPI) == 0, "every thread stores as many pieces, in pairs");
            sx = nrows / RPI;  // the act_s word above may be skipped: not counted
            const int c = bt % CH;
            const uint32_t a0 = lds_addr(stg + (bt / CH) * BNA + c * 16);
            uint8_t* const g0 = p.act + (size_t)(cur.blk * BB + bt / CH) * p.F + cur.nt * BNA + c * 16;
            for (int it = 0; it < nrows / RPI; it += 2) {
              u32x4_t v0, v1;
              lds_read2_b128<RPI * BNA>(a0 + (uint32_t)(it * RPI * BNA), v0, v1);
              *reinterpret_cast<u32x4_t*>(g0 + (size_t)(it * RPI) * p.F) = v0;
              *reinterpret_cast<u32x4_t*>(g0 + (size_t)((it + 1) * RPI) * p.F) = v1;
            }
          }
        } else {
          rows.store(p, lds, cur.nt * BNW, tid);
        }
      }
      if (!more) break;
      if (!PF) {
        lds_barrier();  // every wave is done reading the staged tile
        nx = setup(jn);
      }
      cur = nx;
      pre = PF && nx.ok;
      jn = jnn;
    }
  }
  // the last workgroup to finish leaves the counters at zero for the next
  // launch (every workgroup has made its last take before it counts itself)
  if (dyn && tid == 0 && atomicAdd(p.queue + 8, 1) == (int)gridDim.x - 1) {
#pragma unroll
    for (int x = 0; x < 9; ++x) p.queue[x] = 0;
  }
}

// ---------------------------------------------------------------------------
// Stream kernel (BLOCK_M = 16, decode).  A weight element is used by at most
// the 16 rows of one block, so the kernel is a weight stream: what decides
// its speed is that every CU gets an even share of the weight bytes and keeps
// enough of them in flight.
//
// Tile: 16 padded rows x NC = 16 * FN weight rows.  GEMM1: FN = 1 holds 8
// gate rows (C columns 0-7) and the matching 8 up rows (C columns 8-15); an
// even FN holds FN/2 fragments of gate rows, then FN/2 of up rows; either way
// SwiGLU column j of the tile takes gate column j and up column NC/2 + j.
// GEMM2: NC output columns.  The 8 waves of a workgroup split the K steps
// (one MFMA each) into 8 near-equal contiguous runs; a wave issues the loads
// of S steps at once, then multiplies them (the other waves of the SIMD keep
// the memory pipe busy meanwhile).  A rows of padding slots are not loaded.
// The 8 partial tiles are added in LDS in wave order.  GEMM1 writes SwiGLU
// rows as bf16 (BF16) or fp32 (FP8, MX: their requantisation groups span
// several tiles, so requant_act_kernel quantises the rows afterwards).
// Steps loaded at once: SOp::S, halved for FP8 with 4 fragments (VGPRs).
template <int F, int FN>
constexpr int stream_steps() {
  return (F == F_FP8 && FN == 4) ? SOp<F>::S / 2 : SOp<F>::S;
}

template <int F, int FN, int S>
struct SChunk {
  typename SOp<F>::A a[S];
  typename SOp<F>::B b[FN][S];
  float as[S][4];   // FP8: A scales of C rows 4g .. 4g+3
  float ws[FN][S];  // FP8: weight block scale of this lane's C column
  int sa[S];        // MX: e8m0 of A row r, K block g
  int sb[FN][S];    // MX: e8m0 of weight row r, K block g
};

// Waves per stream workgroup and (0: chosen per shape) fragments per tile;
// compile-time tuning knobs.
#ifndef MOE_STREAM_WAVES
#define MOE_STREAM_WAVES 4
#endif
#ifndef MOE_STREAM_FN
#define MOE_STREAM_FN 0
#endif
constexpr int kStreamWaves = MOE_STREAM_WAVES;
// Waves per tiled (BLOCK_M >= 64, bf16) workgroup: 4 (2 x 2) or 8 (2 x 4).
#ifndef MOE_TILED_WAVES
#define MOE_TILED_WAVES 8
#endif

template <int F, bool G1, int FN>
__global__ __launch_bounds__(64 * kStreamWaves) void gemm_stream(GemmP p) {
  using O = SOp<F>;
  constexpr int SK = O::SK, S = stream_steps<F, FN>();
  constexpr int NC = FN * 16;                // weight rows (C columns) per tile
  constexpr int BNO = G1 ? NC / 2 : NC;      // output columns per tile
  static_assert(!G1 || FN == 1 || FN % 2 == 0, "GEMM1 needs FN = 1 or even");
  extern __shared__ float red_lds[];         // [kStreamWaves][16][NC + 1]
  auto red = reinterpret_cast<float(*)[16][NC + 1]>(red_lds);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int K = G1 ? p.H : p.F;
  const int N = G1 ? p.F : p.H;
  const int ntn = N / BNO;
  const int nblk = *p.npp / 16;
  const int64_t n_valid = (int64_t)nblk * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int ks = K / SK;                                  // MFMA steps over K
  const int st0 = wave * ks / kStreamWaves;               // this wave's steps [st0, st1)
  const int nst = (wave + 1) * ks / kStreamWaves - st0;
  const int rowbytes_a = K * (F == F_BF16 ? 2 : 1);
  const int rowbytes_b = (F == F_MX) ? K / 2 : K * (F == F_BF16 ? 2 : 1);
  const uint8_t* asrc = G1 ? p.x : p.act;
  const uint8_t* wsrc = G1 ? p.w13 : p.w2;
  const size_t erows = G1 ? (size_t)2 * p.F : (size_t)p.H;

  for (int64_t it = blockIdx.x; it < 8 * per; it += gridDim.x) {
    const int64_t L = xcd_tile(it, per);
    if (L >= n_valid) continue;
    const int blk = (int)(L / ntn);
    const int nt = (int)(L % ntn);
    // uniform; readfirstlane keeps the weight descriptor in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(p.block_expert[blk]);
    const int sid = p.sorted_ids[blk * 16 + r];
    const bool aval = sid < p.A;
    const int arow_i = G1 ? (aval ? sid / p.k : 0) : blk * 16 + r;
    const uint8_t* arow = asrc + (size_t)arow_i * rowbytes_a;
    size_t wr[FN];  // weight row (in [E * erows]) of this lane's C column, per fragment
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      int lrow;
      if (G1 && FN == 1)
        lrow = r < 8 ? nt * 8 + r : p.F + nt * 8 + (r - 8);
      else if (G1)
        lrow = fn < FN / 2 ? nt * BNO + fn * 16 + r : p.F + nt * BNO + (fn - FN / 2) * 16 + r;
      else
        lrow = nt * NC + fn * 16 + r;
      wr[fn] = (size_t)e * erows + lrow;
    }
    // FP8: A rows of the C rows 4g .. 4g+3 (their scales)
    int orow[4];
    bool ook[4];
    if (F == F_FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s4 = p.sorted_ids[blk * 16 + 4 * g + i];
        ook[i] = s4 < p.A;
        orow[i] = G1 ? (ook[i] ? s4 / p.k : 0) : blk * 16 + 4 * g + i;
      }
    }

    f32x4_t acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < nst; c0 += S) {
      SChunk<F, FN, S> ch;
      // ---- issue the loads of steps c0 .. c0 + S - 1
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if (c0 + s >= nst) break;
        const int kb = st0 + c0 + s;  // global step index
        if constexpr (F == F_BF16) {
          if (aval)
            ch.a[s] = *reinterpret_cast<const bf16x8_t*>(arow + (size_t)kb * 64 + g * 16);
          else
            ch.a[s] = bf16x8_t{};
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            ch.b[fn][s] = *reinterpret_cast<const bf16x8_t*>(wsrc + wr[fn] * rowbytes_b + (size_t)kb * 64 + g * 16);
        } else if constexpr (F == F_FP8) {
          const float* xsf = static_cast<const float*>(G1 ? p.xs : p.act_s);
          const float* wsf = static_cast<const float*>(G1 ? p.w13_s : p.w2_s);
          const int kblocks = K / 128;
          if (aval)
            ch.a[s] = ld_f8_op(arow + (size_t)kb * 128, g);
          else
            ch.a[s] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < 4; ++i) ch.as[s][i] = ook[i] ? xsf[(size_t)orow[i] * kblocks + kb] : 0.f;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            ch.b[fn][s] = ld_f8_op(wsrc + wr[fn] * rowbytes_b + (size_t)kb * 128, g);
            const size_t wsrow = (wr[fn] / erows) * (erows / 128) + (wr[fn] % erows) / 128;
            ch.ws[fn][s] = wsf[wsrow * kblocks + kb];
          }
        } else {
          const uint8_t* xse = static_cast<const uint8_t*>(G1 ? p.xs : p.act_s);
          const uint8_t* wse = static_cast<const uint8_t*>(G1 ? p.w13_s : p.w2_s);
          const int sblocks = K / 32;
          if (aval) {
            ch.a[s] = ld_f8_op(arow + (size_t)kb * 128, g);
            ch.sa[s] = (int)xse[(size_t)arow_i * sblocks + kb * 4 + g];
          } else {
            ch.a[s] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
            ch.sa[s] = 127;
          }
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            ch.b[fn][s] = *reinterpret_cast<const i32x4_t*>(wsrc + wr[fn] * rowbytes_b + (size_t)kb * 64 + g * 16);
            ch.sb[fn][s] = (int)wse[wr[fn] * sblocks + kb * 4 + g];
          }
        }
      }
      // ---- multiply them, in K order
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if (c0 + s >= nst) break;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          if constexpr (F == F_BF16) {
            acc[fn] = mfma_16x16x32_bf16(ch.a[s], ch.b[fn][s], acc[fn]);
          } else if constexpr (F == F_FP8) {
            const f32x4_t t = mfma_f8(ch.a[s], ch.b[fn][s]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[fn][i] = __builtin_fmaf(t[i], ch.as[s][i] * ch.ws[fn][s], acc[fn][i]);
          } else {
            const i32x4_t v = ch.b[fn][s];
            acc[fn] = mfma_mx(ch.a[s], i32x8_t{v[0], v[1], v[2], v[3], 0, 0, 0, 0}, acc[fn], ch.sa[s], ch.sb[fn][s]);
          }
        }
      }
    }

#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][4 * g + i][fn * 16 + r] = acc[fn][i];
    __syncthreads();

    // ---- epilogue: the 8 partial tiles added in wave order; valid rows only
    for (int idx = threadIdx.x; idx < 16 * BNO; idx += 64 * kStreamWaves) {
      const int row = idx / BNO;
      const int col = idx % BNO;
      const int rsid = p.sorted_ids[blk * 16 + row];
      if (rsid >= p.A) continue;
      if (G1) {
        float gs = red[0][row][col], us = red[0][row][BNO + col];
#pragma unroll
        for (int w = 1; w < kStreamWaves; ++w) {
          gs += red[w][row][col];
          us += red[w][row][BNO + col];
        }
        const float v = swiglu(gs, us, p.lim);
        const size_t o = (size_t)(blk * 16 + row) * p.F + nt * BNO + col;
        if (F == F_BF16)
          reinterpret_cast<uint16_t*>(p.act)[o] = (uint16_t)f32_to_bf16_bits(v);
        else
          p.act32[o] = v;
      } else {
        float s0 = red[0][row][col];
#pragma unroll
        for (int w = 1; w < kStreamWaves; ++w) s0 += red[w][row][col];
        p.out[(size_t)rsid * p.H + nt * NC + col] = (uint16_t)f32_to_bf16_bits(s0);
      }
    }
    __syncthreads();
  }
}

// Requantisation of the fp32 SwiGLU rows the stream GEMM1 wrote (FP8: e4m3
// with scale amax/448 per 128 columns; MX: e4m3 with the e8m0 scale
// pow2_at_least(amax/448) per 32), valid padded rows only.  One workgroup per
// row, each thread 8 consecutive columns.
template <int F>
__global__ __launch_bounds__(256) void requant_act_kernel(GemmP p) {
  const int lane = threadIdx.x & 63;
  const int nrows = *p.npp;
  for (int row = blockIdx.x; row < nrows; row += gridDim.x) {
    if (p.sorted_ids[row] >= p.A) continue;
    for (int c = threadIdx.x * 8; c < p.F; c += 256 * 8) {
      const float4 v0 = *reinterpret_cast<const float4*>(p.act32 + (size_t)row * p.F + c);
      const float4 v1 = *reinterpret_cast<const float4*>(p.act32 + (size_t)row * p.F + c + 4);
      const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
      constexpr int GL = (F == F_FP8) ? 16 : 4;  // lanes per scale group
#pragma unroll
      for (int off = 1; off < GL; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
      float g[8];
      if (F == F_FP8) {
        const float sc = fp8_group_scale(m);
        if ((lane & 15) == 0) static_cast<float*>(p.act_s)[(size_t)row * (p.F / 128) + c / 128] = sc;
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = fp8_scaled(f[i], sc);
      } else {
        const uint32_t code = mx_group_code(m);
        const float inv = e8m0_inv(code);
        if ((lane & 3) == 0) static_cast<uint8_t*>(p.act_s)[(size_t)row * (p.F / 32) + c / 32] = (uint8_t)code;
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = clamp448(f[i] * inv);
      }
      uint2 q;
      q.x = pack4_e4m3(g[0], g[1], g[2], g[3]);
      q.y = pack4_e4m3(g[4], g[5], g[6], g[7]);
      *reinterpret_cast<uint2*>(p.act + (size_t)row * p.F + c) = q;
    }
  }
}

// Fragments per tile for the stream kernels: the widest tile (fewest re-reads
// of the A rows) that still leaves >= 2048 tiles (8 per CU) for the expected
// number of experts touched, E (1 - (1 - k/E)^T).
int stream_fn(int T, int k, int E, int N, bool g1) {
  if (MOE_STREAM_FN != 0) return MOE_STREAM_FN;
  const double touched = E * (1.0 - std::pow(1.0 - (double)k / E, (double)T));
  const int fns[3] = {4, 2, 1};
  for (int fn : fns) {
    const int bno = g1 ? fn * 8 : fn * 16;
    if (N % bno == 0 && touched * (N / bno) >= 2048.0) return fn;
  }
  return 1;
}

// Workgroups of `kernel` that fit on the current device at once (CUs x
// occupancy), as a multiple of 8.  `cache` (one per kernel, indexed by
// device) keeps the answer; concurrent first calls compute the same value,
// so relaxed atomics suffice.
int resident_wgs(const void* kernel, int threads, size_t lds, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    v = (cus * per_cu + 7) / 8 * 8;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int F, bool G1, int FN>
void launch_stream_one(const GemmP& p, int64_t max_blocks, int N, hipStream_t s) {
  constexpr int BNO = G1 ? FN * 8 : FN * 16;
  const size_t lds = (size_t)kStreamWaves * 16 * (FN * 16 + 1) * sizeof(float);
  // every workgroup resident at once: a workgroup that finds no tile exits
  // at once instead of holding a slot that a tile could use
  static std::atomic<int> cache[64];
  const int wgs = resident_wgs(reinterpret_cast<const void*>(&gemm_stream<F, G1, FN>), 64 * kStreamWaves, lds, cache);
  gemm_stream<F, G1, FN><<<tile_grid(max_blocks * (N / BNO), wgs), 64 * kStreamWaves, lds, s>>>(p);
}

template <int F, bool G1, int BM, int BNW, int NS, int NW = 4, int KMX = 1>
moe_status launch_tiled_one(const GemmP& p, int64_t max_tiles, hipStream_t s) {
  using T = Tr<F>;
  constexpr int KSQ = (F == F_MX) ? KMX : 1;  // as in gemm_tiled
  const size_t sc = (F == F_BF16) ? 0 : (size_t)KSQ * ((BM + BNW + 64 * NW - 1) / (64 * NW)) * 64 * NW * 4;
  const size_t lds = (size_t)NS * ((size_t)KSQ * BM * 128 + (size_t)BNW * T::BROW * KSQ + sc);
  // the workgroups resident at once (each loops over tiles)
  static std::atomic<int> cache[64];
  const int wgs =
      resident_wgs(reinterpret_cast<const void*>(&gemm_tiled<F, G1, BM, BNW, NS, NW, KMX>), 64 * NW, lds, cache);
  gemm_tiled<F, G1, BM, BNW, NS, NW, KMX><<<tile_grid(max_tiles, wgs), 64 * NW, lds, s>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

#ifndef MOE_PAIR_WAVES
#define MOE_PAIR_WAVES 8
#endif
template <bool G1, int BB>
moe_status launch_pair_one(const GemmP& p, int64_t max_tiles, hipStream_t s) {
  // one workgroup per CU (the rings are all of LDS at BB = 128), each looping over tiles
  constexpr int NW = MOE_PAIR_WAVES;
  constexpr size_t lds = (size_t)2 * (2 * BB) * 128 + (size_t)3 * 256 * 128;  // A: 2 slots, B: 3 slots
  static std::atomic<int> cache[64];
  const int wgs = resident_wgs(reinterpret_cast<const void*>(&gemm_pair_bf16<G1, NW, BB>), 64 * NW, lds, cache);
  gemm_pair_bf16<G1, NW, BB><<<tile_grid(max_tiles, wgs), 64 * NW, lds, s>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <bool G1, int BB>
moe_status launch_pair_mx_one(const GemmP& p, int64_t max_tiles, hipStream_t s) {
  constexpr size_t lds = (size_t)MOE_MX_A_SLOTS * (2 * BB * 128) + (size_t)MOE_MX_B_SLOTS * 256 * 64 +
                        2 * 512 * 16;  // A, weight and (2) scale-group slots
  static std::atomic<int> cache[64];
  const int wgs = resident_wgs(reinterpret_cast<const void*>(&gemm_pair_mx<G1, BB>), 512, lds, cache);
  gemm_pair_mx<G1, BB><<<tile_grid(max_tiles, wgs), 512, lds, s>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <int F>
moe_status launch_gemm_fmt(const FfnArgs& a, int which, hipStream_t s) {
  GemmP p;
  const bool q = F != F_BF16;
  p.x = static_cast<const uint8_t*>(q ? a.xq : a.x);
  p.xs = a.xs;
  p.w13 = static_cast<const uint8_t*>(a.w13);
  p.w13_s = a.w13_scale;
  p.w2 = static_cast<const uint8_t*>(a.w2);
  p.w2_s = a.w2_scale;
  p.sorted_ids = a.sorted_ids;
  p.block_expert = a.block_expert;
  p.npp = a.num_post_padded;
  p.act = static_cast<uint8_t*>(a.act);
  p.act_s = a.act_s;
  p.act32 = static_cast<float*>(a.act32);
  p.out = static_cast<uint16_t*>(a.out);
  p.pairs = static_cast<const int32_t*>(a.pairs);
  p.queue = reinterpret_cast<int*>(static_cast<char*>(a.ctrl) + kTileQueueOffset);
  p.lim = a.swiglu_limit;
  p.H = a.H; p.F = a.F; p.k = a.k; p.A = a.T * a.k;
  const int64_t mb = align_max_blocks(a.T, a.k, a.E, a.block_m);
  if (a.block_m == 16) {
    const int N = which == 1 ? a.F : a.H;
    const int fn = stream_fn(a.T, a.k, a.E, N, which == 1);
    if (which == 1) {
      if (fn == 4) launch_stream_one<F, true, 4>(p, mb, N, s);
      else if (fn == 2) launch_stream_one<F, true, 2>(p, mb, N, s);
      else launch_stream_one<F, true, 1>(p, mb, N, s);
      MOE_CHECK_LAUNCH();
      if (F != F_BF16) {
        requant_act_kernel<F><<<tile_grid(align_max_padded(a.T, a.k, a.E, 16), 4096), 256, 0, s>>>(p);
        MOE_CHECK_LAUNCH();
      }
    } else {
      if (fn == 4) launch_stream_one<F, false, 4>(p, mb, N, s);
      else if (fn == 2) launch_stream_one<F, false, 2>(p, mb, N, s);
      else launch_stream_one<F, false, 1>(p, mb, N, s);
      MOE_CHECK_LAUNCH();
    }
    return MOE_OK;
  }
  const int64_t t1 = mb * (a.F / 128), t2 = mb * (a.H / 128);
  // 8 waves (2 x 4) for bf16 and fp8 at BLOCK_M >= 64; MX keeps 4 (measured:
  // 8 waves were 7 % faster for the fp8 DeepSeek-V3 prefill, and no faster
  // or slower for MX)
  constexpr int NW = (F == F_MX) ? 4 : MOE_TILED_WAVES;
  switch (a.block_m) {
    case 32:  // MX: 256-wide K steps (measured: faster here; at 64 and 128 rows slower, one workgroup per CU)
      if constexpr (F == F_BF16) {
        if (a.pairs) {
          if (which == 1) return launch_pair_one<true, 32>(p, t1, s);
          if (a.H % 256 == 0) return launch_pair_one<false, 32>(p, t2 / 2, s);
        }
      }
      if (which == 1) return launch_tiled_one<F, true, 32, 256, 3, 4, 2>(p, t1, s);
      // MX GEMM2: 256 output columns once that still leaves >= 2048 tiles
      // (measured: DSV4 T=512 layer 770 -> 753 us; with fewer tiles, as for
      // bf16 GLM T=8, the CUs go short: 509 -> 529 us)
      if constexpr (F == F_MX)
        if (a.H % 256 == 0 && t2 / 2 >= 2048) return launch_tiled_one<F, false, 32, 256, 3, 4, 2>(p, t2 / 2, s);
      return launch_tiled_one<F, false, 32, 128, 3, 4, 2>(p, t2, s);
    case 64:
      if constexpr (F == F_BF16) {
        if (a.pairs) {
          if (which == 1) return launch_pair_one<true, 64>(p, t1, s);
          if (a.H % 256 == 0) return launch_pair_one<false, 64>(p, t2 / 2, s);
        }
      }
      if constexpr (F == F_MX) {
        if (a.pairs) {
          if (which == 1) return launch_pair_mx_one<true, 64>(p, t1, s);
          if (a.H % 256 == 0) return launch_pair_mx_one<false, 64>(p, t2 / 2, s);
        }
      }
      if (which == 1) return launch_tiled_one<F, true, 64, 256, (F == F_BF16 ? 4 : 3), NW>(p, t1, s);
      // GEMM2 in 256 output columns when H allows (bf16 and fp8; measured,
      // fp8 DSV3 T=1024: 805 -> 745 us against 128 columns)
      if constexpr (F == F_BF16 || F == F_FP8)
        if (a.H % 256 == 0) return launch_tiled_one<F, false, 64, 256, 3, NW>(p, t2 / 2, s);
      return launch_tiled_one<F, false, 64, 128, 3, NW>(p, t2, s);
    case 128:
      if constexpr (F == F_BF16) {
        if (a.pairs) {
          if (which == 1) return launch_pair_one<true, 128>(p, t1, s);
          if (a.H % 256 == 0) return launch_pair_one<false, 128>(p, t2 / 2, s);
        }
      }
      if constexpr (F == F_MX) {
        if (a.pairs) {
          if (which == 1) return launch_pair_mx_one<true, 128>(p, t1, s);
          if (a.H % 256 == 0) return launch_pair_mx_one<false, 128>(p, t2 / 2, s);
        }
      }
      if (which == 1) return launch_tiled_one<F, true, 128, 256, 3, NW>(p, t1, s);
      // (fp8 DSV3 T=2048: 958 -> 845 us against 128 columns)
      if constexpr (F == F_BF16 || F == F_FP8)
        if (a.H % 256 == 0) return launch_tiled_one<F, false, 128, 256, 3, NW>(p, t2 / 2, s);
      return launch_tiled_one<F, false, 128, 128, 3, NW>(p, t2, s);
  }
  return MOE_E_INVAL;
}

}  // namespace

#ifndef MOE_PAIRED_TILES
#define MOE_PAIRED_TILES 1
#endif
bool ffn_paired(int wformat, int block_m, int T, int k, int E) {
  if (!MOE_PAIRED_TILES) return false;
  if (block_m == 64 || block_m == 128) return wformat == MOE_W_BF16 || wformat == MOE_W_MXFP4;
  // bf16 at 32 rows: pairs of 32-row blocks once the experts average two
  // rows or more and the alignment has a launch of its own (above 64
  // assignments).  Measured (cold layers, against the 32-row tiled kernel):
  // GLM T=512 2078 -> 1849 us (the selection bias gives some experts many
  // blocks, each of which the tiled kernel copies the weights for), Qwen3
  // T=64 level; GLM T=8 (single blocks) 527 -> 549 us and the toy T=16
  // layer (an extra pair-table launch) 25 -> 30 us are why the cuts exist.
  return wformat == MOE_W_BF16 && block_m == 32 && (int64_t)T * k >= 2 * (int64_t)E && (int64_t)T * k > 64;
}

moe_status launch_pair_table(const FfnArgs& a, hipStream_t s) {
  pair_table_kernel<<<1, 1024, 0, s>>>(a.block_expert, a.num_post_padded, a.block_m, static_cast<int32_t*>(a.pairs));
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

moe_status launch_gemm_bf16(const FfnArgs& a, int which, hipStream_t s) { return launch_gemm_fmt<F_BF16>(a, which, s); }
moe_status launch_gemm_fp8(const FfnArgs& a, int which, hipStream_t s) { return launch_gemm_fmt<F_FP8>(a, which, s); }
moe_status launch_gemm_mxfp4(const FfnArgs& a, int which, hipStream_t s) { return launch_gemm_fmt<F_MX>(a, which, s); }

moe_status launch_quant_x(const FfnArgs& a, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  uint8_t* xq = static_cast<uint8_t*>(a.xq);
  if (a.wformat == MOE_W_FP8_BLOCK128)
    quant_x_kernel<F_FP8><<<a.T, 256, 0, s>>>(x, xq, a.xs, a.H);
  else if (a.wformat == MOE_W_MXFP4)
    quant_x_kernel<F_MX><<<a.T, 256, 0, s>>>(x, xq, a.xs, a.H);
  else
    return MOE_OK;
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace moe
