// Matrix-core issue-rate probe (moe_probe_mfma): the rate a full chip of
// independent MFMA chains reaches for each instruction the grouped GEMMs
// issue, the ceiling their MFMA fractions are read against.
#include "common.h"

namespace moe {
namespace {

constexpr int kProbeWaves = 4;  // waves per workgroup

// One wave keeps NA independent accumulators and cycles through them
// `iters` times; the operands are register constants, so nothing but the
// matrix cores is exercised.  KIND: 0 bf16 16x16x32, 1 bf16 32x32x16,
// 2 e4m3 x e4m3, 3 e4m3 x e2m1, 4 e2m1 x e2m1 (16x16x128 with e8m0 scales).
template <int KIND, int NA>
__global__ __launch_bounds__(64 * kProbeWaves) void mfma_probe_kernel(float* sink, int iters) {
  const int t = threadIdx.x;
  float s = 0.f;
  if constexpr (KIND == 0 || KIND == 1) {
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(float)((t + i) % 7 - 3);
      b[i] = (__bf16)(float)((t * 3 + i) % 5 - 2);
    }
    if constexpr (KIND == 0) {
      f32x4_t c[NA];
#pragma unroll
      for (int j = 0; j < NA; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < NA; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NA; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    } else {
      f32x16_t c[NA];
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) c[j][q] = 0.f;
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < NA; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) s += c[j][q];
    }
  } else {
    constexpr int FA = KIND == 4 ? 4 : 0;  // operand format codes: 0 e4m3, 4 e2m1
    constexpr int FB = KIND == 2 ? 0 : 4;
    i32x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (FA == 4 && i >= 4) ? 0 : 0x3A3A3A3A + t + i;
      b[i] = (FB == 4 && i >= 4) ? 0 : 0x2C2C2C2C + 3 * t + i;
    }
    f32x4_t c[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NA; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], FA, FB, 0, 127, 0, 127);
#pragma unroll
    for (int j = 0; j < NA; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  }
  sink[(size_t)blockIdx.x * (64 * kProbeWaves) + t] = s;
}

template <int KIND>
hipError_t launch_probe(int accs, int grid, int iters, float* sink, hipStream_t stream) {
  const dim3 g(grid), b(64 * kProbeWaves);
  switch (accs) {
    case 4: mfma_probe_kernel<KIND, 4><<<g, b, 0, stream>>>(sink, iters); break;
    case 8: mfma_probe_kernel<KIND, 8><<<g, b, 0, stream>>>(sink, iters); break;
    case 16:
      if constexpr (KIND == 1) return hipErrorInvalidValue;  // 256 accumulator registers
      else mfma_probe_kernel<KIND, 16><<<g, b, 0, stream>>>(sink, iters);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_probe_mfma_sink_len(int grid) { return grid > 0 ? (size_t)grid * 64 * moe::kProbeWaves : 0; }

extern "C" moe_status moe_probe_mfma(int kind, int accs, int grid, int iters, float* sink, hipStream_t stream) {
  if (!sink || grid <= 0 || iters <= 0 || (accs != 4 && accs != 8 && accs != 16)) return MOE_E_INVAL;
  if (kind == 1 && accs == 16) return MOE_E_INVAL;  // 256 accumulator registers
  hipError_t e;
  switch (kind) {
    case 0: e = moe::launch_probe<0>(accs, grid, iters, sink, stream); break;
    case 1: e = moe::launch_probe<1>(accs, grid, iters, sink, stream); break;
    case 2: e = moe::launch_probe<2>(accs, grid, iters, sink, stream); break;
    case 3: e = moe::launch_probe<3>(accs, grid, iters, sink, stream); break;
    case 4: e = moe::launch_probe<4>(accs, grid, iters, sink, stream); break;
    default: return MOE_E_INVAL;
  }
  return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}
