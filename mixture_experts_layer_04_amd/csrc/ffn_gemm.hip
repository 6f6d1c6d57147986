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
//  * BLOCK_M = 16 ("stream", decode): the weights are the traffic.  The 4
//    waves of a workgroup split K into quarters and load operands straight
//    into VGPRs (a weight element is used once); the quarters are reduced in
//    LDS in a fixed order before the epilogue.
//  * BLOCK_M >= 32 ("tiled", prefill): 2 x 2 waves, A (BLOCK_M rows) and B
//    tiles copied straight into a 3-stage LDS ring two K steps (128 bytes of
//    K per row each) ahead of the multiply; one barrier per step; the output
//    tile leaves through LDS as whole rows.
// Tiles are visited in a grid-stride loop bounded by the padded length read
// on the device (no workgroup is launched for blocks that do not exist), in
// an order that keeps the blocks sharing a weight tile on one XCD.

#include "common.h"
#include "launch.h"

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
  uint16_t* out;          // [T*k, H] bf16
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
  static constexpr int KSTEP = 128;
  static constexpr int BROW = 64;
  static constexpr int BNA_STREAM = 32;
};

__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.f + expf(-g)) * u; }

// e4m3 (OCP) of v, v already within [-448, 448]; round to nearest even
__device__ __forceinline__ uint32_t to_e4m3(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFu;
}
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
  return (uint32_t)hi;
}
__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// Power-of-two scale >= v (v > 0) as its e8m0 code; 127 (2^0) for v == 0.
__device__ __forceinline__ uint32_t e8m0_at_least(float v) {
  if (!(v > 0.f)) return 127u;
  const uint32_t u = __float_as_uint(v);
  uint32_t e = (u >> 23) & 0xFFu;
  if (e == 0u) return 1u;                 // below the normal range: smallest code used
  if ((u & 0x7FFFFFu) != 0u) e += 1u;     // not a power of two: round up
  return e > 254u ? 254u : e;
}
__device__ __forceinline__ float e8m0_value(uint32_t code) { return __uint_as_float(code << 23); }
__device__ __forceinline__ float e8m0_inv(uint32_t code) { return __uint_as_float((254u - code) << 23); }

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
    float inv;
    if (F == F_FP8) {
      const float s = m > 0.f ? m / 448.f : 1.f;
      inv = 1.f / s;
      if ((lane & 15) == 0) static_cast<float*>(xs)[(size_t)t * (H / 128) + h / 128] = s;
    } else {
      const uint32_t c = e8m0_at_least(m / 448.f);
      inv = e8m0_inv(c);
      if ((lane & 3) == 0) static_cast<uint8_t*>(xs)[(size_t)t * (H / 32) + h / 32] = (uint8_t)c;
    }
    uint2 q;
    q.x = pack4_e4m3(clamp448(f[0] * inv), clamp448(f[1] * inv), clamp448(f[2] * inv), clamp448(f[3] * inv));
    q.y = pack4_e4m3(clamp448(f[4] * inv), clamp448(f[5] * inv), clamp448(f[6] * inv), clamp448(f[7] * inv));
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
// columns).  Waves 2 x 2: wave (wm, wn) owns rows [wm*BM/2, +BM/2) and weight
// rows: GEMM1 gate [wn*BNW/4, +BNW/4) and up [BNW/2 + wn*BNW/4, +BNW/4);
// GEMM2 [wn*BNW/2, +BNW/2).
//
// K steps of 128 bytes per row are copied global -> LDS with
// global_load_lds_dwordx4 (no VGPR staging) into a ring of NS stages, NS - 1
// steps ahead of the multiply; one barrier per step.  Inside a stage a row's
// 16-byte chunk c sits at slot c ^ f(row) (f(row) = (row / (16 / chunks per
// row)) mod chunks per row), so the 16 rows one MFMA operand read touches
// fall in 16 different bank groups.  The epilogue stages the output tile in
// LDS and writes whole rows with 16-byte stores.
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

__device__ __forceinline__ void g2lds16(const uint8_t* g, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((gvoid_t*)g, (lvoid_t*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* g, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds((gvoid_t*)g, (lvoid_t*)lds_dst, 4, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier for the copy pipeline: each wave has already waited for
// its own copies of the step (wait_vm), so no memory fence is needed, and a
// fence would also wait for the copies still in flight for later steps.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
template <int CPR>
__device__ __forceinline__ int swz(int c, int row) {
  return c ^ ((row / (16 / CPR)) & (CPR - 1));
}

template <int F, bool G1, int BM, int BNW, int NS>
__global__ __launch_bounds__(256) void gemm_tiled(GemmP p) {
  using T = Tr<F>;
  constexpr int CPRB = T::BROW / 16;   // 16-byte chunks per B row and step
  constexpr int ASZ = BM * 128;
  constexpr int BSZ = BNW * T::BROW;
  constexpr int FM = BM / 32;
  constexpr int FN = BNW / 32;
  constexpr int LA = BM / 32;          // A copy instructions per wave per step
  constexpr int LB = BNW * CPRB / 256; // B copy instructions per wave per step
  // scales (FP8, MX): one 4-byte word per tile row (A: the row's scale(s) of
  // the step, B: the weight row's) copied with the data; every wave issues
  // the same number of copies, the slots past BM + BNW are never read
  constexpr int LSC = (F == F_BF16) ? 0 : (BM + BNW + 255) / 256;
  constexpr int LS = LA + LB + LSC;
  constexpr int SCSZ = LSC * 256 * 4;
  constexpr int SSZ = ASZ + BSZ + SCSZ;
  constexpr int D = NS - 1;            // steps in flight ahead of the multiply
  static_assert(LS * (D > 1 ? D - 1 : 1) <= 63, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int K = G1 ? p.H : p.F;
  const int N = G1 ? p.F : p.H;
  const int BNO = G1 ? BNW / 2 : BNW;
  const int ntn = N / BNO;
  const int nblk = *p.npp / BM;
  const int64_t n_valid = (int64_t)nblk * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int nk = K / T::KSTEP;
  const int rowbytes_a = K * T::AB;
  const int rowbytes_b = (F == F_MX) ? K / 2 : K * T::AB;
  const uint8_t* asrc = G1 ? p.x : p.act;
  const uint8_t* wsrc = G1 ? p.w13 : p.w2;
  const size_t erows = G1 ? (size_t)2 * p.F : (size_t)p.H;

  // tile-local weight row of fragment fn of this wave
  auto frag_lrow = [&](int fn) {
    return G1 ? (fn < FN / 2 ? wn * (BNW / 4) + fn * 16 : BNW / 2 + wn * (BNW / 4) + (fn - FN / 2) * 16)
              : wn * (BNW / 2) + fn * 16;
  };
  auto weight_row = [&](int nt, int lrow) {
    if (G1) return lrow < BNW / 2 ? nt * (BNW / 2) + lrow : p.F + nt * (BNW / 2) + (lrow - BNW / 2);
    return nt * BNW + lrow;
  };

  for (int64_t it = blockIdx.x; it < 8 * per; it += gridDim.x) {
    const int64_t L = xcd_tile(it, per);
    if (L >= n_valid) continue;
    const int blk = (int)(L % nblk);
    const int nt = (int)(L / nblk);
    const int e = p.block_expert[blk];

    // per-lane global sources of the copy instructions
    const uint8_t* ag[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = wave * (BM / 4) + 8 * i + (lane >> 3);
      bool v;
      const int src = a_row_index<G1>(p, blk, BM, row, v);  // padding rows read token 0; never used
      ag[i] = asrc + (size_t)src * rowbytes_a + 16 * swz<8>(lane & 7, row);
    }
    const uint8_t* bg[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = (wave * LB + i) * (64 / CPRB) + lane / CPRB;
      bg[i] = wsrc + ((size_t)e * erows + weight_row(nt, row)) * rowbytes_b + 16 * swz<CPRB>(lane % CPRB, row);
    }
    // scale words: slot q = (i * 4 + wave) * 64 + lane of copy i; q < BM: A
    // row q, q < BM + BNW: B row q - BM.  Per step the source advances by
    // sc_step bytes.
    const uint8_t* scg[LSC > 0 ? LSC : 1];
    int sc_step[LSC > 0 ? LSC : 1];
    if (F != F_BF16) {
      const int kblocks = K / 128;  // FP8: one fp32 scale per 128 K; MX: 4 e8m0 per 128 K
#pragma unroll
      for (int i = 0; i < LSC; ++i) {
        const int q = (i * 4 + wave) * 64 + lane;
        if (q < BM) {
          bool v;
          const int src = a_row_index<G1>(p, blk, BM, q, v);
          if (F == F_FP8) {
            scg[i] = static_cast<const uint8_t*>(G1 ? p.xs : p.act_s) + ((size_t)src * kblocks) * 4;
            sc_step[i] = 4;
          } else {
            scg[i] = static_cast<const uint8_t*>(G1 ? p.xs : p.act_s) + (size_t)src * (K / 32);
            sc_step[i] = 4;
          }
        } else {
          const int lrow = q < BM + BNW ? q - BM : 0;
          const int wr = weight_row(nt, lrow);
          if (F == F_FP8) {
            scg[i] = static_cast<const uint8_t*>(G1 ? p.w13_s : p.w2_s) +
                     (((size_t)e * (erows / 128) + wr / 128) * kblocks) * 4;
            sc_step[i] = 4;
          } else {
            scg[i] = static_cast<const uint8_t*>(G1 ? p.w13_s : p.w2_s) + ((size_t)e * erows + wr) * (K / 32);
            sc_step[i] = 4;
          }
        }
      }
    }
    // copy step s into ring slot `slot`
    auto issue = [&](int s, int slot) {
      uint8_t* st = lds + slot * SSZ;
#pragma unroll
      for (int i = 0; i < LA; ++i) g2lds16(ag[i] + (size_t)s * 128, st + (wave * (BM / 4) + 8 * i) * 128);
#pragma unroll
      for (int i = 0; i < LB; ++i)
        g2lds16(bg[i] + (size_t)s * T::BROW, st + ASZ + (wave * LB + i) * (64 / CPRB) * T::BROW);
#pragma unroll
      for (int i = 0; i < LSC; ++i) g2lds4(scg[i] + (size_t)s * sc_step[i], st + ASZ + BSZ + (i * 4 + wave) * 256);
    };

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // the previous tile is done with LDS
    // Every step issues exactly one step of copies (the last D - 1 steps copy
    // step nk - 1 again into ring slots that no later step reads), so the
    // number of copies in flight is always (D - 1) * LS at the wait below and
    // the compiler's own waits for the scale loads stay exact.
#pragma unroll
    for (int s = 0; s < D; ++s) issue(s < nk ? s : nk - 1, s % NS);

    for (int s = 0; s < nk; ++s) {
      wait_vm<(D - 1) * LS>();
      barrier_no_fence();
      issue(s + D < nk ? s + D : nk - 1, (s + D) % NS);

      const uint8_t* As = lds + (s % NS) * SSZ;
      const uint8_t* Bs = As + ASZ;
      const uint8_t* Ss = Bs + BSZ;  // scale words of the step
      if (F == F_BF16) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8_t af[FM], bfr[FN];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            const int rr = wm * (BM / 2) + fm * 16 + r;
            af[fm] = *reinterpret_cast<const bf16x8_t*>(As + rr * 128 + 16 * swz<8>(ks * 4 + g, rr));
          }
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int rr = frag_lrow(fn) + r;
            bfr[fn] = *reinterpret_cast<const bf16x8_t*>(Bs + rr * 128 + 16 * swz<8>(ks * 4 + g, rr));
          }
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn]);
        }
      } else {
        i32x8_t af[FM];
        float as_[FM][4];
        int sa[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          if (F == F_FP8) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              as_[fm][i] = reinterpret_cast<const float*>(Ss)[wm * (BM / 2) + fm * 16 + 4 * g + i];
          } else {
            sa[fm] = (int)Ss[(wm * (BM / 2) + fm * 16 + r) * 4 + g];
          }
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          const int rr = wm * (BM / 2) + fm * 16 + r;
          const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(As + rr * 128 + 16 * swz<8>(g, rr));
          const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(As + rr * 128 + 16 * swz<8>(4 + g, rr));
          af[fm] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int rr = frag_lrow(fn) + r;
          if (F == F_FP8) {
            const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(Bs + rr * 128 + 16 * swz<8>(g, rr));
            const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(Bs + rr * 128 + 16 * swz<8>(4 + g, rr));
            const i32x8_t bfr = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const float wsc = reinterpret_cast<const float*>(Ss)[BM + frag_lrow(fn)];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
              const f32x4_t t = mfma_f8(af[fm], bfr);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[fm][fn][i] = __builtin_fmaf(t[i], as_[fm][i] * wsc, acc[fm][fn][i]);
            }
          } else {
            const i32x4_t v = *reinterpret_cast<const i32x4_t*>(Bs + rr * 64 + 16 * swz<4>(g, rr));
            const i32x8_t bfr = {v[0], v[1], v[2], v[3], 0, 0, 0, 0};
            const int sb = (int)Ss[(BM + rr) * 4 + g];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fm][fn] = mfma_mx(af[fm], bfr, acc[fm][fn], sa[fm], sb);
          }
        }
      }
    }
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
          for (int i = 0; i < 4; ++i) v[fm][fa][i] = swiglu(acc[fm][fa][i], acc[fm][fa + FA][i]);
      const int lcol0 = wn * (BNA / 2);  // first tile column of this wave
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
        float* xch = reinterpret_cast<float*>(lds + BM * BNA);  // [2][BM] after the byte tile
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float mm = 0.f;
#pragma unroll
            for (int fa = 0; fa < FA; ++fa) mm = fmaxf(mm, fabsf(v[fm][fa][i]));
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, kWave));
            if (r == 0) xch[wn * BM + wm * (BM / 2) + fm * 16 + 4 * g + i] = mm;
          }
        __syncthreads();
        float* act_s = static_cast<float*>(p.act_s);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int lr = wm * (BM / 2) + fm * 16 + 4 * g + i;
            const float amax = fmaxf(xch[lr], xch[BM + lr]);
            const float sc = amax > 0.f ? amax / 448.f : 1.f;
            const float inv = 1.f / sc;
            if (wn == 0 && r == 0) act_s[(size_t)(blk * BM + lr) * (p.F / 128) + nt] = sc;
#pragma unroll
            for (int fa = 0; fa < FA; ++fa)
              lds[lr * BNA + lcol0 + fa * 16 + r] = (uint8_t)to_e4m3(clamp448(v[fm][fa][i] * inv));
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
              float mm = fmaxf(fabsf(v[fm][2 * gp][i]), fabsf(v[fm][2 * gp + 1][i]));
#pragma unroll
              for (int off = 1; off < 16; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, kWave));
              const uint32_t c = e8m0_at_least(mm / 448.f);
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
      for (int idx = tid; idx < BM * CH; idx += 256) {
        const int lr = idx / CH;
        const int c = idx % CH;
        const uint4 val = *reinterpret_cast<const uint4*>(lds + lr * RB + c * 16);
        *reinterpret_cast<uint4*>(p.act + ((size_t)(blk * BM + lr) * p.F + nt * BNA) * T::AB + c * 16) = val;
      }
    } else {
      uint16_t* st = reinterpret_cast<uint16_t*>(lds);  // [BM][BNW]
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            st[(wm * (BM / 2) + fm * 16 + 4 * g + i) * BNW + wn * (BNW / 2) + fn * 16 + r] =
                (uint16_t)f32_to_bf16_bits(acc[fm][fn][i]);
      __syncthreads();
      constexpr int CH = BNW * 2 / 16;
      for (int idx = tid; idx < BM * CH; idx += 256) {
        const int lr = idx / CH;
        const int c = idx % CH;
        const int sid = p.sorted_ids[blk * BM + lr];
        if (sid >= p.A) continue;
        const uint4 val = *reinterpret_cast<const uint4*>(lds + lr * BNW * 2 + c * 16);
        *reinterpret_cast<uint4*>(p.out + (size_t)sid * p.H + nt * BNW + c * 8) = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stream kernel (BLOCK_M = 16).  Tile: 16 rows x BNA SwiGLU columns (GEMM1:
// BNA gate + BNA up weight rows; BNA = 16 / 128 / 32 for BF16 / FP8 / MX so
// that a requantisation group lies inside one tile) or 16 rows x 16 output
// columns (GEMM2).  The 4 waves split K into quarters.
template <int F, bool G1>
__global__ __launch_bounds__(256) void gemm_stream(GemmP p) {
  using T = Tr<F>;
  constexpr int BM = 16;
  constexpr int BNA = G1 ? T::BNA_STREAM : 16;   // output columns per tile
  constexpr int FN = G1 ? 2 * BNA / 16 : 1;       // weight fragments per wave
  constexpr int NCOL = FN * 16;                   // weight rows per tile
  extern __shared__ float red_lds[];              // [4][BM][NCOL + 1]
  auto red = reinterpret_cast<float(*)[BM][NCOL + 1]>(red_lds);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int K = G1 ? p.H : p.F;
  const int N = G1 ? p.F : p.H;
  const int ntn = N / BNA;
  const int nblk = *p.npp / BM;
  const int64_t n_valid = (int64_t)nblk * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int kq = K / 4;                         // elements per wave
  const int nsteps = kq / T::KSTEP;
  const int rowbytes_a = K * T::AB;
  const int rowbytes_b = (F == F_MX) ? K / 2 : K * T::AB;
  const uint8_t* asrc = G1 ? p.x : p.act;
  const uint8_t* wsrc = G1 ? p.w13 : p.w2;
  const size_t erows = G1 ? (size_t)2 * p.F : (size_t)p.H;

  for (int64_t it = blockIdx.x; it < 8 * per; it += gridDim.x) {
    const int64_t L = xcd_tile(it, per);
    if (L >= n_valid) continue;
    const int blk = (int)(L / ntn);
    const int nt = (int)(L % ntn);
    const int e = p.block_expert[blk];
    bool aval;
    const int asrc_row = a_row_index<G1>(p, blk, BM, r, aval);
    const uint8_t* arow = asrc + (size_t)asrc_row * rowbytes_a;
    int wrow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      if (G1)
        wrow[fn] = fn < FN / 2 ? nt * BNA + fn * 16 : p.F + nt * BNA + (fn - FN / 2) * 16;
      else
        wrow[fn] = nt * 16;
    }
    f32x4_t acc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int k0 = wave * kq;  // first K element of this wave

    if (F == F_BF16) {
      for (int kk = 0; kk < kq; kk += 32) {
        bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + (size_t)(k0 + kk + 8 * g) * 2);
        if (!aval) a = bf16x8_t{};
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const uint8_t* b = wsrc + ((size_t)e * erows + wrow[fn] + r) * rowbytes_b + (size_t)(k0 + kk + 8 * g) * 2;
          acc[fn] = mfma_16x16x32_bf16(a, *reinterpret_cast<const bf16x8_t*>(b), acc[fn]);
        }
      }
    } else if (F == F_FP8) {
      const float* xsf = static_cast<const float*>(G1 ? p.xs : p.act_s);
      const float* wsf = static_cast<const float*>(G1 ? p.w13_s : p.w2_s);
      const int kblocks = K / 128;
      const size_t erows_blk = erows / 128;
      // A row scales of this lane's 4 output rows
      int orow[4];
      bool ook[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bool v;
        orow[i] = a_row_index<G1>(p, blk, BM, 4 * g + i, v);
        ook[i] = v;
      }
      for (int st = 0; st < nsteps; ++st) {
        const int kb = k0 / 128 + st;
        i32x8_t a = ld_f8_op(arow + (size_t)kb * 128, g);
        if (!aval) a = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        float as_[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) as_[i] = ook[i] ? xsf[(size_t)orow[i] * kblocks + kb] : 0.f;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const uint8_t* b = wsrc + ((size_t)e * erows + wrow[fn] + r) * rowbytes_b + (size_t)kb * 128;
          const f32x4_t t = mfma_f8(a, ld_f8_op(b, g));
          const float wsc = wsf[((size_t)e * erows_blk + wrow[fn] / 128) * kblocks + kb];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[fn][i] = __builtin_fmaf(t[i], as_[i] * wsc, acc[fn][i]);
        }
      }
    } else {  // F_MX
      const uint8_t* xse = static_cast<const uint8_t*>(G1 ? p.xs : p.act_s);
      const uint8_t* wse = static_cast<const uint8_t*>(G1 ? p.w13_s : p.w2_s);
      const int sblocks = K / 32;
      for (int st = 0; st < nsteps; ++st) {
        const int kb = k0 / 128 + st;
        i32x8_t a = ld_f8_op(arow + (size_t)kb * 128, g);
        const int sa = aval ? (int)xse[(size_t)asrc_row * sblocks + kb * 4 + g] : 127;
        if (!aval) a = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const size_t wr = (size_t)e * erows + wrow[fn] + r;
          const i32x8_t b = ld_f4_op(wsrc + wr * rowbytes_b + (size_t)kb * 64, g);
          const int sb = (int)wse[wr * sblocks + kb * 4 + g];
          acc[fn] = mfma_mx(a, b, acc[fn], sa, sb);
        }
      }
    }

#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][4 * g + i][fn * 16 + r] = acc[fn][i];
    __syncthreads();

    // epilogue: 256 threads, 16 per row; each thread BNA / 16 columns
    {
      const int row = threadIdx.x >> 4;
      const int c16 = threadIdx.x & 15;
      if (G1) {
        constexpr int CPT = BNA / 16;  // SwiGLU columns per thread
        float v[CPT];
        float mm = 0.f;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const int col = c16 * CPT + j;  // column inside the tile
          float gs = red[0][row][col], us = red[0][row][BNA + col];
#pragma unroll
          for (int w = 1; w < 4; ++w) {
            gs += red[w][row][col];
            us += red[w][row][BNA + col];
          }
          v[j] = swiglu(gs, us);
          mm = fmaxf(mm, fabsf(v[j]));
        }
        const size_t prow = (size_t)blk * BM + row;
        const int colg = nt * BNA + c16 * CPT;
        if (F == F_BF16) {
          reinterpret_cast<uint16_t*>(p.act)[prow * p.F + colg] = (uint16_t)f32_to_bf16_bits(v[0]);
        } else {
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, kWave));
          float inv;
          if (F == F_FP8) {
            const float sc = mm > 0.f ? mm / 448.f : 1.f;
            inv = 1.f / sc;
            if (c16 == 0) static_cast<float*>(p.act_s)[prow * (p.F / 128) + nt] = sc;
          } else {
            const uint32_t c = e8m0_at_least(mm / 448.f);
            inv = e8m0_inv(c);
            if (c16 == 0) static_cast<uint8_t*>(p.act_s)[prow * (p.F / 32) + nt] = (uint8_t)c;
          }
#pragma unroll
          for (int j = 0; j < CPT; ++j) p.act[prow * p.F + colg + j] = (uint8_t)to_e4m3(clamp448(v[j] * inv));
        }
      } else {
        float s0 = red[0][row][c16];
        s0 += red[1][row][c16];
        s0 += red[2][row][c16];
        s0 += red[3][row][c16];
        const int sid = p.sorted_ids[blk * BM + row];
        if (sid < p.A) p.out[(size_t)sid * p.H + nt * 16 + c16] = (uint16_t)f32_to_bf16_bits(s0);
      }
    }
    __syncthreads();
  }
}

template <int F, bool G1, int BM, int BNW, int NS>
moe_status launch_tiled_one(const GemmP& p, int64_t max_tiles, hipStream_t s) {
  using T = Tr<F>;
  const size_t sc = (F == F_BF16) ? 0 : (size_t)((BM + BNW + 255) / 256) * 1024;
  const size_t lds = (size_t)NS * ((size_t)BM * 128 + (size_t)BNW * T::BROW + sc);
  gemm_tiled<F, G1, BM, BNW, NS><<<tile_grid(max_tiles, 512), 256, lds, s>>>(p);
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
  p.out = static_cast<uint16_t*>(a.out);
  p.H = a.H; p.F = a.F; p.k = a.k; p.A = a.T * a.k;
  const int64_t mb = align_max_blocks(a.T, a.k, a.E, a.block_m);
  if (a.block_m == 16) {
    constexpr int NCOL1 = 2 * Tr<F>::BNA_STREAM;
    if (which == 1)
      gemm_stream<F, true><<<tile_grid(mb * (a.F / Tr<F>::BNA_STREAM), 2048), 256, 4 * 16 * (NCOL1 + 1) * 4, s>>>(p);
    else
      gemm_stream<F, false><<<tile_grid(mb * (a.H / 16), 2048), 256, 4 * 16 * (16 + 1) * 4, s>>>(p);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  const int64_t t1 = mb * (a.F / 128), t2 = mb * (a.H / 128);
  switch (a.block_m) {
    case 32: return which == 1 ? launch_tiled_one<F, true, 32, 256, 3>(p, t1, s) : launch_tiled_one<F, false, 32, 128, 3>(p, t2, s);
    case 64: return which == 1 ? launch_tiled_one<F, true, 64, 256, 3>(p, t1, s) : launch_tiled_one<F, false, 64, 128, 3>(p, t2, s);
    case 128: return which == 1 ? launch_tiled_one<F, true, 128, 256, 3>(p, t1, s) : launch_tiled_one<F, false, 128, 128, 3>(p, t2, s);
  }
  return MOE_E_INVAL;
}

}  // namespace

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
