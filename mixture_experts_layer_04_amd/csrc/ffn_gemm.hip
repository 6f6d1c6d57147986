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
//    tiles double-buffered in LDS, 128 bytes of K per row per step, the next
//    step's global loads in flight while the current step is multiplied; one
//    barrier per step.
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
template <int F, bool G1, int BM, int BNW>
__global__ __launch_bounds__(256) void gemm_tiled(GemmP p) {
  using T = Tr<F>;
  constexpr int LDA = 128 + 16;                 // LDS bytes per A row
  constexpr int LDB = T::BROW + 16;             // LDS bytes per B row
  constexpr int ASZ = BM * LDA;
  constexpr int BSZ = BNW * LDB;
  constexpr int FM = BM / 32;
  constexpr int FN = BNW / 32;
  constexpr int A_CH = BM * 8 / 256;            // 16-byte pieces per thread
  constexpr int B_PR = T::BROW / 16;            // pieces per B row
  constexpr int B_CH = BNW * B_PR / 256;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int K = G1 ? p.H : p.F;                 // in elements
  const int N = G1 ? p.F : p.H;                 // output columns
  const int BNO = G1 ? BNW / 2 : BNW;
  const int ntn = N / BNO;
  const int nblk = *p.npp / BM;
  const int64_t n_valid = (int64_t)nblk * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int nk = K / T::KSTEP;
  const int rowbytes_a = K * T::AB;             // bytes per A row in global memory
  const int rowbytes_b = (F == F_MX) ? K / 2 : K * T::AB;
  const uint8_t* asrc = G1 ? p.x : p.act;
  const uint8_t* wsrc = G1 ? p.w13 : p.w2;

  for (int64_t it = blockIdx.x; it < 8 * per; it += gridDim.x) {
    const int64_t L = xcd_tile(it, per);
    if (L >= n_valid) continue;
    const int blk = (int)(L % nblk);
    const int nt = (int)(L / nblk);
    const int e = p.block_expert[blk];

    // global sources of this thread's pieces
    const uint8_t* ap[A_CH];
    bool av[A_CH];
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch >> 3;
      bool v;
      const int src = a_row_index<G1>(p, blk, BM, row, v);
      av[c] = v;
      ap[c] = asrc + (size_t)src * rowbytes_a + (ch & 7) * 16;
    }
    const uint8_t* bp[B_CH];
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch / B_PR;
      int wrow;
      if (G1)
        wrow = row < BNW / 2 ? nt * (BNW / 2) + row : p.F + nt * (BNW / 2) + (row - BNW / 2);
      else
        wrow = nt * BNW + row;
      const size_t erows = G1 ? (size_t)2 * p.F : (size_t)p.H;
      bp[c] = wsrc + ((size_t)e * erows + wrow) * rowbytes_b + (ch % B_PR) * 16;
    }

    // rows of this wave's fragments (for the epilogue and the scales)
    int arow_src[FM][4];
    bool arow_ok[FM][4];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bool v;
        arow_src[fm][i] = a_row_index<G1>(p, blk, BM, wm * (BM / 2) + fm * 16 + 4 * g + i, v);
        arow_ok[fm][i] = v;
      }
    // MX: the A scale of lane (r, g) is that of row r of each fragment
    int mx_arow[FM];
    bool mx_aok[FM];
    if (F == F_MX) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        bool v;
        mx_arow[fm] = a_row_index<G1>(p, blk, BM, wm * (BM / 2) + fm * 16 + r, v);
        mx_aok[fm] = v;
      }
    }
    // weight row of fragment fn, column r (for MX B scales) and the first
    // weight row of each fragment (for FP8 block scales)
    int frow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      int lrow;  // row inside the tile
      if (G1)
        lrow = fn < FN / 2 ? wn * (BNW / 4) + fn * 16 : BNW / 2 + wn * (BNW / 4) + (fn - FN / 2) * 16;
      else
        lrow = wn * (BNW / 2) + fn * 16;
      if (G1)
        frow[fn] = lrow < BNW / 2 ? nt * (BNW / 2) + lrow : p.F + nt * (BNW / 2) + (lrow - BNW / 2);
      else
        frow[fn] = nt * BNW + lrow;
    }

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[A_CH], rb[B_CH];
    auto gload = [&](int s) {
      const int offa = s * 128;
      const int offb = s * T::BROW;
#pragma unroll
      for (int c = 0; c < A_CH; ++c) ra[c] = *reinterpret_cast<const uint4*>(ap[c] + offa);
#pragma unroll
      for (int c = 0; c < B_CH; ++c) rb[c] = *reinterpret_cast<const uint4*>(bp[c] + offb);
    };
    auto sstore = [&](int buf) {
      uint8_t* As = lds + buf * (ASZ + BSZ);
      uint8_t* Bs = As + ASZ;
#pragma unroll
      for (int c = 0; c < A_CH; ++c) {
        const int ch = tid + 256 * c;
        uint4 v = ra[c];
        if (!av[c]) v = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(As + (ch >> 3) * LDA + (ch & 7) * 16) = v;
      }
#pragma unroll
      for (int c = 0; c < B_CH; ++c) {
        const int ch = tid + 256 * c;
        *reinterpret_cast<uint4*>(Bs + (ch / B_PR) * LDB + (ch % B_PR) * 16) = rb[c];
      }
    };

    __syncthreads();  // the previous tile's last reads of LDS are done
    gload(0);
    sstore(0);
    if (nk > 1) gload(1);
    __syncthreads();

    for (int s = 0; s < nk; ++s) {
      if (s + 1 < nk) sstore((s + 1) & 1);
      if (s + 2 < nk) gload(s + 2);
      const uint8_t* As = lds + (s & 1) * (ASZ + BSZ);
      const uint8_t* Bs = As + ASZ;
      if (F == F_BF16) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8_t af[FM], bfr[FN];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) af[fm] = ld_bf16_op(As + (wm * (BM / 2) + fm * 16 + r) * LDA, ks, g);
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int lrow = G1 ? (fn < FN / 2 ? wn * (BNW / 4) + fn * 16 : BNW / 2 + wn * (BNW / 4) + (fn - FN / 2) * 16)
                                : wn * (BNW / 2) + fn * 16;
            bfr[fn] = ld_bf16_op(Bs + (lrow + r) * LDB, ks, g);
          }
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn]);
        }
      } else if (F == F_FP8) {
        // fp32 block scales of this 128-wide K block
        const float* xsf = static_cast<const float*>(G1 ? p.xs : p.act_s);
        const int kblocks = K / 128;
        float as_[FM][4];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) as_[fm][i] = xsf[(size_t)arow_src[fm][i] * kblocks + s];
        const float* wsf = static_cast<const float*>(G1 ? p.w13_s : p.w2_s);
        const size_t erows_blk = G1 ? (size_t)(2 * p.F / 128) : (size_t)(p.H / 128);
        i32x8_t af[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) af[fm] = ld_f8_op(As + (wm * (BM / 2) + fm * 16 + r) * LDA, g);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int lrow = G1 ? (fn < FN / 2 ? wn * (BNW / 4) + fn * 16 : BNW / 2 + wn * (BNW / 4) + (fn - FN / 2) * 16)
                              : wn * (BNW / 2) + fn * 16;
          const i32x8_t bfr = ld_f8_op(Bs + (lrow + r) * LDB, g);
          const float wsc = wsf[((size_t)e * erows_blk + frow[fn] / 128) * kblocks + s];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            const f32x4_t t = mfma_f8(af[fm], bfr);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[fm][fn][i] = __builtin_fmaf(t[i], as_[fm][i] * wsc, acc[fm][fn][i]);
          }
        }
      } else {  // F_MX
        const uint8_t* xse = static_cast<const uint8_t*>(G1 ? p.xs : p.act_s);
        const uint8_t* wse = static_cast<const uint8_t*>(G1 ? p.w13_s : p.w2_s);
        const int sblocks = K / 32;
        const size_t erows = G1 ? (size_t)2 * p.F : (size_t)p.H;
        i32x8_t af[FM];
        int sa[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          af[fm] = ld_f8_op(As + (wm * (BM / 2) + fm * 16 + r) * LDA, g);
          sa[fm] = mx_aok[fm] ? (int)xse[(size_t)mx_arow[fm] * sblocks + s * 4 + g] : 127;
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int lrow = G1 ? (fn < FN / 2 ? wn * (BNW / 4) + fn * 16 : BNW / 2 + wn * (BNW / 4) + (fn - FN / 2) * 16)
                              : wn * (BNW / 2) + fn * 16;
          const i32x8_t bfr = ld_f4_op(Bs + (lrow + r) * LDB, g);
          const int sb = (int)wse[((size_t)e * erows + frow[fn] + r) * sblocks + s * 4 + g];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) acc[fm][fn] = mfma_mx(af[fm], bfr, acc[fm][fn], sa[fm], sb);
        }
      }
      __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    if (G1) {
      constexpr int FA = FN / 2;  // SwiGLU fragments of this wave
      float v[FM][FA][4];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fa = 0; fa < FA; ++fa)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[fm][fa][i] = swiglu(acc[fm][fa][i], acc[fm][fa + FA][i]);
      const int col0 = nt * (BNW / 2) + wn * (BNW / 4);  // first SwiGLU column of this wave
      if (F == F_BF16) {
        uint16_t* act = reinterpret_cast<uint16_t*>(p.act);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = blk * BM + wm * (BM / 2) + fm * 16 + 4 * g + i;
#pragma unroll
            for (int fa = 0; fa < FA; ++fa)
              act[(size_t)row * p.F + col0 + fa * 16 + r] = (uint16_t)f32_to_bf16_bits(v[fm][fa][i]);
          }
      } else if (F == F_FP8) {
        // amax over the tile's BNW/2 = 128 columns of each row (two waves)
        float* xch = reinterpret_cast<float*>(lds);  // [2][BM]
        float m[FM][4];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float mm = 0.f;
#pragma unroll
            for (int fa = 0; fa < FA; ++fa) mm = fmaxf(mm, fabsf(v[fm][fa][i]));
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, kWave));
            m[fm][i] = mm;
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
            const int row = blk * BM + lr;
            if (wn == 0 && r == 0) act_s[(size_t)row * (p.F / 128) + nt] = sc;
#pragma unroll
            for (int fa = 0; fa < FA; ++fa)
              p.act[(size_t)row * p.F + col0 + fa * 16 + r] = (uint8_t)to_e4m3(clamp448(v[fm][fa][i] * inv));
          }
        __syncthreads();
      } else {  // F_MX: groups of 32 columns = fragment pairs of this wave
        uint8_t* act_s = static_cast<uint8_t*>(p.act_s);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = blk * BM + wm * (BM / 2) + fm * 16 + 4 * g + i;
#pragma unroll
            for (int gp = 0; gp < FA / 2; ++gp) {
              float mm = fmaxf(fabsf(v[fm][2 * gp][i]), fabsf(v[fm][2 * gp + 1][i]));
#pragma unroll
              for (int off = 1; off < 16; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, kWave));
              const uint32_t c = e8m0_at_least(mm / 448.f);
              const float inv = e8m0_inv(c);
              const int col = col0 + gp * 32;
              if (r == 0) act_s[(size_t)row * (p.F / 32) + col / 32] = (uint8_t)c;
              p.act[(size_t)row * p.F + col + r] = (uint8_t)to_e4m3(clamp448(v[fm][2 * gp][i] * inv));
              p.act[(size_t)row * p.F + col + 16 + r] = (uint8_t)to_e4m3(clamp448(v[fm][2 * gp + 1][i] * inv));
            }
          }
      }
    } else {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (!arow_ok[fm][i]) continue;
          const int row = blk * BM + wm * (BM / 2) + fm * 16 + 4 * g + i;
          const int sid = p.sorted_ids[row];
          if (sid >= p.A) continue;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            p.out[(size_t)sid * p.H + nt * BNW + wn * (BNW / 2) + fn * 16 + r] =
                (uint16_t)f32_to_bf16_bits(acc[fm][fn][i]);
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

template <int F, bool G1, int BM, int BNW>
moe_status launch_tiled_one(const GemmP& p, int64_t max_tiles, hipStream_t s) {
  using T = Tr<F>;
  const size_t lds = 2 * ((size_t)BM * (128 + 16) + (size_t)BNW * (T::BROW + 16));
  gemm_tiled<F, G1, BM, BNW><<<tile_grid(max_tiles, 512), 256, lds, s>>>(p);
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
    case 32: return which == 1 ? launch_tiled_one<F, true, 32, 256>(p, t1, s) : launch_tiled_one<F, false, 32, 128>(p, t2, s);
    case 64: return which == 1 ? launch_tiled_one<F, true, 64, 256>(p, t1, s) : launch_tiled_one<F, false, 64, 128>(p, t2, s);
    case 128: return which == 1 ? launch_tiled_one<F, true, 128, 256>(p, t1, s) : launch_tiled_one<F, false, 128, 128>(p, t2, s);
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
