// Grouped expert GEMMs for bf16 weights: GEMM1 (+SwiGLU epilogue) and GEMM2.
//
// [Kernels] "The fused expert GEMM": each tile owns one block of BLOCK_M
// rows, reads that block's single expert from the block table, gathers its
// activation rows through sorted_ids / k (rows at or past T*k are padding and
// contribute zeros), and GEMM1's gate and up columns produce silu(g) * u in
// the epilogue ([MegaMoE] §3.5: the activation is the tail of the GEMM1
// task).  GEMM2 reads the SwiGLU rows in block order and writes each real row
// to its assignment slot of the [T*k, H] output; padding rows are dropped.
//
// Both operands are K-contiguous (x [T, H] against w13 [E, 2F, H]; act
// [rows, F] against w2 [E, H, F]), which is the native operand order of the
// v_mfma_f32_16x16x32_bf16 instruction: lane l supplies row (l % 16) and the
// 8 K-values at 8 * (l / 16) of each 32-wide K step, and receives rows
// 4 * (l / 16) + i, column l % 16 of the 16x16 fp32 result.
//
// Two tile shapes (one template family):
//  * BLOCK_M = 16 ("stream", decode): the weights are the traffic.  A
//    workgroup's 4 waves split K into quarters and load their operands
//    straight from global memory into VGPRs (a weight element is used once,
//    LDS staging would only add latency); the quarters are reduced in LDS in
//    a fixed order.  Small output tiles (16 columns) give enough workgroups
//    to keep every CU streaming.
//  * BLOCK_M >= 32 ("tiled", prefill): 2 x 2 waves share LDS tiles of A
//    (BLOCK_M x 64) and B (128 weight rows x 64); the next K step is
//    prefetched into VGPRs while the current one is multiplied.
// Tiles are visited in a grid-stride loop bounded by the padded length read
// on the device, so no workgroup is launched for blocks that do not exist.

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

struct GemmP {
  const uint16_t* x;
  const uint16_t* w13;
  const uint16_t* w2;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* npp;
  uint16_t* act;
  uint16_t* out;
  int H, F, k, A;
};

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// ----------------------------------------------------------------------------
// BLOCK_M = 16, split-K over the 4 waves of a workgroup.
// GEMM1 tile: 16 rows x 16 SwiGLU columns (16 gate + 16 up weight rows).
// GEMM2 tile: 16 rows x 16 output columns.
template <bool G1>
__global__ __launch_bounds__(256) void gemm_stream_bf16(GemmP p) {
  constexpr int BM = 16;
  constexpr int NPART = G1 ? 2 : 1;
  __shared__ float red[4][NPART][16][17];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int K = G1 ? p.H : p.F;
  const int N = G1 ? p.F : p.H;
  const int ntn = N / 16;
  const int nblk = *p.npp / BM;
  const int64_t n_valid = (int64_t)nblk * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int kw = K >> 2;

  for (int64_t i = blockIdx.x; i < 8 * per; i += gridDim.x) {
    const int64_t L = xcd_tile(i, per);
    if (L >= n_valid) continue;
    const int blk = (int)(L / ntn);
    const int nt = (int)(L % ntn);
    const int e = p.block_expert[blk];
    const uint16_t* arow;
    bool aval = true;
    if (G1) {
      const int sid = p.sorted_ids[blk * BM + r];
      aval = sid < p.A;
      arow = p.x + (size_t)(aval ? sid / p.k : 0) * p.H;
    } else {
      arow = p.act + (size_t)(blk * BM + r) * p.F;
    }
    const uint16_t* b0;
    const uint16_t* b1 = nullptr;
    if (G1) {
      b0 = p.w13 + ((size_t)e * 2 * p.F + nt * 16 + r) * p.H;
      b1 = b0 + (size_t)p.F * p.H;
    } else {
      b0 = p.w2 + ((size_t)e * p.H + nt * 16 + r) * p.F;
    }
    const int kb = wave * kw + q * 8;
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
    f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int kk = 0; kk < kw; kk += 32) {
      bf16x8_t a = ld_bf16x8(arow + kb + kk);
      if (!aval) a = bf16x8_t{};
      const bf16x8_t w0 = ld_bf16x8(b0 + kb + kk);
      acc0 = mfma_16x16x32_bf16(a, w0, acc0);
      if (G1) {
        const bf16x8_t w1 = ld_bf16x8(b1 + kb + kk);
        acc1 = mfma_16x16x32_bf16(a, w1, acc1);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      red[wave][0][4 * q + j][r] = acc0[j];
      if (G1) red[wave][NPART - 1][4 * q + j][r] = acc1[j];
    }
    __syncthreads();
    {
      const int row = threadIdx.x >> 4;
      const int col = threadIdx.x & 15;
      float s0 = red[0][0][row][col];
      s0 += red[1][0][row][col];
      s0 += red[2][0][row][col];
      s0 += red[3][0][row][col];
      if (G1) {
        float s1 = red[0][NPART - 1][row][col];
        s1 += red[1][NPART - 1][row][col];
        s1 += red[2][NPART - 1][row][col];
        s1 += red[3][NPART - 1][row][col];
        p.act[(size_t)(blk * BM + row) * p.F + nt * 16 + col] = (uint16_t)f32_to_bf16_bits(silu_mul(s0, s1));
      } else {
        const int sid = p.sorted_ids[blk * BM + row];
        if (sid < p.A) p.out[(size_t)sid * p.H + nt * 16 + col] = (uint16_t)f32_to_bf16_bits(s0);
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// BLOCK_M in {32, 64, 128}: LDS-tiled, 2 x 2 waves.
// GEMM1 tile: BM rows x 64 SwiGLU columns (weight rows: 64 gate then 64 up).
// GEMM2 tile: BM rows x 128 output columns.
template <int BM, bool G1>
__global__ __launch_bounds__(256) void gemm_tiled_bf16(GemmP p) {
  constexpr int BK = 64;
  constexpr int LD = BK + 8;  // padded row (elements): 144 B rows spread the banks
  constexpr int BNW = 128;    // weight rows per tile
  constexpr int FM = BM / 32; // 16-row fragments per wave
  constexpr int A_CH = BM * 8 / 256;
  constexpr int B_CH = BNW * 8 / 256;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BNW * LD];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int K = G1 ? p.H : p.F;
  const int N = G1 ? p.F : p.H;
  const int BNO = G1 ? 64 : 128;
  const int ntn = N / BNO;
  const int nblk = *p.npp / BM;
  const int64_t n_valid = (int64_t)nblk * ntn;
  const int64_t per = (n_valid + 7) >> 3;
  const int nk = K / BK;

  for (int64_t i = blockIdx.x; i < 8 * per; i += gridDim.x) {
    const int64_t L = xcd_tile(i, per);
    if (L >= n_valid) continue;
    const int blk = (int)(L % nblk);  // consecutive tiles: same weight tile
    const int nt = (int)(L / nblk);
    const int e = p.block_expert[blk];

    const uint16_t* ap[A_CH];
    bool av[A_CH];
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch >> 3;
      const int col = (ch & 7) * 8;
      if (G1) {
        const int sid = p.sorted_ids[blk * BM + row];
        av[c] = sid < p.A;
        ap[c] = p.x + (size_t)(av[c] ? sid / p.k : 0) * p.H + col;
      } else {
        av[c] = true;
        ap[c] = p.act + (size_t)(blk * BM + row) * p.F + col;
      }
    }
    const uint16_t* bp[B_CH];
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch >> 3;
      const int col = (ch & 7) * 8;
      if (G1) {
        const int wrow = row < 64 ? nt * 64 + row : p.F + nt * 64 + (row - 64);
        bp[c] = p.w13 + ((size_t)e * 2 * p.F + wrow) * p.H + col;
      } else {
        bp[c] = p.w2 + ((size_t)e * p.H + nt * 128 + row) * p.F + col;
      }
    }

    f32x4_t acc[FM][4];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[A_CH], rb[B_CH];
#pragma unroll
    for (int c = 0; c < A_CH; ++c) ra[c] = *reinterpret_cast<const uint4*>(ap[c]);
#pragma unroll
    for (int c = 0; c < B_CH; ++c) rb[c] = *reinterpret_cast<const uint4*>(bp[c]);

    for (int kt = 0; kt < nk; ++kt) {
      __syncthreads();
#pragma unroll
      for (int c = 0; c < A_CH; ++c) {
        const int ch = tid + 256 * c;
        uint4 v = ra[c];
        if (!av[c]) v = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&As[(ch >> 3) * LD + (ch & 7) * 8]) = v;
      }
#pragma unroll
      for (int c = 0; c < B_CH; ++c) {
        const int ch = tid + 256 * c;
        *reinterpret_cast<uint4*>(&Bs[(ch >> 3) * LD + (ch & 7) * 8]) = rb[c];
      }
      __syncthreads();
      if (kt + 1 < nk) {
        const int off = (kt + 1) * BK;
#pragma unroll
        for (int c = 0; c < A_CH; ++c) ra[c] = *reinterpret_cast<const uint4*>(ap[c] + off);
#pragma unroll
        for (int c = 0; c < B_CH; ++c) rb[c] = *reinterpret_cast<const uint4*>(bp[c] + off);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t af[FM], bfr[4];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          af[fm] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * (BM / 2) + fm * 16 + r) * LD + ks * 32 + q * 8]);
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          const int nrow = G1 ? ((fn < 2) ? wn * 32 + fn * 16 : 64 + wn * 32 + (fn - 2) * 16) : wn * 64 + fn * 16;
          bfr[fn] = *reinterpret_cast<const bf16x8_t*>(&Bs[(nrow + r) * LD + ks * 32 + q * 8]);
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < 4; ++fn) acc[fm][fn] = mfma_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn]);
      }
    }

    if (G1) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int row = wm * (BM / 2) + fm * 16 + 4 * q + ii;
            const int col = nt * 64 + wn * 32 + j * 16 + r;
            p.act[(size_t)(blk * BM + row) * p.F + col] =
                (uint16_t)f32_to_bf16_bits(silu_mul(acc[fm][j][ii], acc[fm][j + 2][ii]));
          }
    } else {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = wm * (BM / 2) + fm * 16 + 4 * q + ii;
          const int sid = p.sorted_ids[blk * BM + row];
          if (sid < p.A) {
#pragma unroll
            for (int fn = 0; fn < 4; ++fn) {
              const int col = nt * 128 + wn * 64 + fn * 16 + r;
              p.out[(size_t)sid * p.H + col] = (uint16_t)f32_to_bf16_bits(acc[fm][fn][ii]);
            }
          }
        }
    }
  }
}

template <int BM>
moe_status launch_tiled(const GemmP& p, int which, int64_t max_tiles1, int64_t max_tiles2, hipStream_t s) {
  if (which == 1)
    gemm_tiled_bf16<BM, true><<<tile_grid(max_tiles1, 1024), 256, 0, s>>>(p);
  else
    gemm_tiled_bf16<BM, false><<<tile_grid(max_tiles2, 1024), 256, 0, s>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace

moe_status launch_gemm_bf16(const FfnArgs& a, int which, hipStream_t s) {
  GemmP p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.w13 = static_cast<const uint16_t*>(a.w13);
  p.w2 = static_cast<const uint16_t*>(a.w2);
  p.sorted_ids = a.sorted_ids;
  p.block_expert = a.block_expert;
  p.npp = a.num_post_padded;
  p.act = static_cast<uint16_t*>(a.act);
  p.out = static_cast<uint16_t*>(a.out);
  p.H = a.H; p.F = a.F; p.k = a.k; p.A = a.T * a.k;
  const int64_t mb = align_max_blocks(a.T, a.k, a.E, a.block_m);
  switch (a.block_m) {
    case 16: {
      if (which == 1)
        gemm_stream_bf16<true><<<tile_grid(mb * (a.F / 16), 2048), 256, 0, s>>>(p);
      else
        gemm_stream_bf16<false><<<tile_grid(mb * (a.H / 16), 2048), 256, 0, s>>>(p);
      MOE_CHECK_LAUNCH();
      return MOE_OK;
    }
    case 32: return launch_tiled<32>(p, which, mb * (a.F / 64), mb * (a.H / 128), s);
    case 64: return launch_tiled<64>(p, which, mb * (a.F / 64), mb * (a.H / 128), s);
    case 128: return launch_tiled<128>(p, which, mb * (a.F / 64), mb * (a.H / 128), s);
  }
  return MOE_E_INVAL;
}

}  // namespace moe
