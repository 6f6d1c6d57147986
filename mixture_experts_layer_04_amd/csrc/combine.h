// The combine arithmetic of one token and 8 consecutive output columns ([Kernels] "Combine, backward and low precision": a
// per-token gather summing its k rows in a fixed order is deterministic;
// [MegaMoE] §3.7: the slots are added as fp32 in slot order and rounded once).
#pragma once

#include "common.h"

namespace moe {

// y[t, h .. h+7] from out rows t*k + j (bf16 [T*k, H]), ids / w of token t
// (k entries each); slots whose id is outside [0, E) add nothing.  KM = k.
template <int KM>
__device__ __forceinline__ uint4 combine8(const uint16_t* out, const int32_t* ids, const float* w, int t, int h,
                                          int H, int E, int k) {
  uint4 o[KM];  // all k rows in flight at once (read once: non-temporal), then added in slot order
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(out + ((size_t)t * k + j) * H + h));
    o[j] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int e = ids[j];
    if (e < 0 || e >= E) continue;
    const float wj = w[j];
    acc[0] = __builtin_fmaf(wj, bf16_lo(o[j].x), acc[0]);
    acc[1] = __builtin_fmaf(wj, bf16_hi(o[j].x), acc[1]);
    acc[2] = __builtin_fmaf(wj, bf16_lo(o[j].y), acc[2]);
    acc[3] = __builtin_fmaf(wj, bf16_hi(o[j].y), acc[3]);
    acc[4] = __builtin_fmaf(wj, bf16_lo(o[j].z), acc[4]);
    acc[5] = __builtin_fmaf(wj, bf16_hi(o[j].z), acc[5]);
    acc[6] = __builtin_fmaf(wj, bf16_lo(o[j].w), acc[6]);
    acc[7] = __builtin_fmaf(wj, bf16_hi(o[j].w), acc[7]);
  }
  uint4 v;
  v.x = pack_bf16x2(acc[0], acc[1]);
  v.y = pack_bf16x2(acc[2], acc[3]);
  v.z = pack_bf16x2(acc[4], acc[5]);
  v.w = pack_bf16x2(acc[6], acc[7]);
  return v;
}

}  // namespace moe
