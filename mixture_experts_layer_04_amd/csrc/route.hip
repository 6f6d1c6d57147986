// Router: gate logits + scoring + (group limit) + top-k + renormalisation in
// one launch.
//
// [Router] §1.1 (three steps), §1.3 (rank key = score + bias, weight = score),
// §5.3 (one row per wave, k rounds, lowest id wins ties), §8.1 (the GEMV
// wants expert-parallel blocks, the top-k wants row-parallel waves) and §9
// (a token's logits must not depend on its batch).
//
// Layout of the work: blocks tile (expert tile x token tile).  Each wave owns
// EPW experts and computes their fp32 dot products with TPB tokens; lane l
// accumulates the 8-element chunks c = l, l+64, ... of H with fmaf in a
// fixed order, then a butterfly sums the 64 lanes.  The per-(token, expert)
// arithmetic is therefore identical for every T and tile shape.  After its
// logits are stored, each block bumps an agent-scope counter of its token
// tile; the block that arrives last (there is no waiting) runs the selection
// for the tile's tokens, one wave per token, with the E logits held in VGPRs
// (slot s of lane l is expert s*64 + l), and resets the counter to zero.

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

struct RouteParams {
  const uint16_t* x;
  const float* gate;
  const float* bias;
  float* logits;
  unsigned* counters;
  int32_t* ids;
  float* weights;
  int T, H, E, k, n_group, topk_group, scoring, renorm;
  float scale;
  int n_etiles;
};

template <int TPB, int EPW>
__device__ __forceinline__ void gemv_tile(const RouteParams& p, int ttile, int etile) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t0 = ttile * TPB;
  const int e0 = etile * (4 * EPW) + wave * EPW;
  const float* g[EPW];
  const uint16_t* xr[TPB];
#pragma unroll
  for (int i = 0; i < EPW; ++i) g[i] = p.gate + (size_t)min(e0 + i, p.E - 1) * p.H;
#pragma unroll
  for (int j = 0; j < TPB; ++j) xr[j] = p.x + (size_t)min(t0 + j, p.T - 1) * p.H;

  float acc[TPB][EPW];
#pragma unroll
  for (int j = 0; j < TPB; ++j)
#pragma unroll
    for (int i = 0; i < EPW; ++i) acc[j][i] = 0.f;

  const int nchunk = p.H >> 3;
#pragma unroll 2
  for (int c = lane; c < nchunk; c += kWave) {
    float gv[EPW][8];
#pragma unroll
    for (int i = 0; i < EPW; ++i) {
      const float4* gp = reinterpret_cast<const float4*>(g[i] + (size_t)c * 8);
      const float4 a = gp[0];
      const float4 b = gp[1];
      gv[i][0] = a.x; gv[i][1] = a.y; gv[i][2] = a.z; gv[i][3] = a.w;
      gv[i][4] = b.x; gv[i][5] = b.y; gv[i][6] = b.z; gv[i][7] = b.w;
    }
#pragma unroll
    for (int j = 0; j < TPB; ++j) {
      uint4 xv = *reinterpret_cast<const uint4*>(xr[j] + (size_t)c * 8);
      float xf[8] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y),
                     bf16_lo(xv.z), bf16_hi(xv.z), bf16_lo(xv.w), bf16_hi(xv.w)};
#pragma unroll
      for (int i = 0; i < EPW; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[j][i] = __builtin_fmaf(xf[q], gv[i][q], acc[j][i]);
    }
  }
#pragma unroll
  for (int j = 0; j < TPB; ++j)
#pragma unroll
    for (int i = 0; i < EPW; ++i) {
      float v = wave_sum(acc[j][i]);
      if (lane == 0 && t0 + j < p.T && e0 + i < p.E) p.logits[(size_t)(t0 + j) * p.E + e0 + i] = v;
    }
}

template <int SLOTS>
__device__ __forceinline__ void select_token(const RouteParams& p, int t) {
  const int lane = threadIdx.x & 63;
  const float* lg = p.logits + (size_t)t * p.E;
  float key[SLOTS], sc[SLOTS];
  bool ok[SLOTS];
  const float NEG_INF = -__builtin_inff();

  float l[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int e = s * kWave + lane;
    ok[s] = e < p.E;
    l[s] = ok[s] ? lg[e] : NEG_INF;
  }
  if (p.scoring == MOE_SOFTMAX) {
    float m = NEG_INF;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) m = fmaxf(m, l[s]);
    m = wave_max(m);
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      sc[s] = ok[s] ? expf(l[s] - m) : 0.f;
      part += sc[s];
    }
    const float inv = 1.f / wave_sum(part);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      sc[s] = sc[s] * inv;
      key[s] = ok[s] ? sc[s] : NEG_INF;
    }
  } else {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int e = s * kWave + lane;
      sc[s] = 1.f / (1.f + expf(-l[s]));
      const float b = (p.bias != nullptr && ok[s]) ? p.bias[e] : 0.f;
      key[s] = ok[s] ? sc[s] + b : NEG_INF;
    }
  }

  if (p.n_group > 1) {
    // group score = sum of the two largest rank keys of the group
    const int gsize = p.E / p.n_group;
    float my_gs = NEG_INF;
    for (int g = 0; g < p.n_group; ++g) {
      float t1 = NEG_INF, t2 = NEG_INF;
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int e = s * kWave + lane;
        if (ok[s] && e / gsize == g) {
          const float v = key[s];
          if (v > t1) { t2 = t1; t1 = v; } else if (v > t2) { t2 = v; }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float o1 = __shfl_xor(t1, off, kWave);
        const float o2 = __shfl_xor(t2, off, kWave);
        const float n1 = fmaxf(t1, o1);
        const float n2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
        t1 = n1; t2 = n2;
      }
      if (lane == g) my_gs = t1 + t2;
    }
    // keep the topk_group best groups, lowest group id on ties
    uint64_t kept = 0;
    bool g_used = lane >= p.n_group;
    for (int r = 0; r < p.topk_group; ++r) {
      uint64_t v = g_used ? 0ull
                          : (((uint64_t)f32_order_key(my_gs) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)lane));
      v = wave_max_u64(v);
      const int g = (int)(0xFFFFFFFFu - (uint32_t)v);
      kept |= 1ull << g;
      if (lane == g) g_used = true;
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const int e = s * kWave + lane;
      if (ok[s] && !((kept >> (e / gsize)) & 1ull)) ok[s] = false;
    }
  }

  // k rounds of wave arg-max on (key descending, id ascending)
  int sel_id = 0;
  float sel_s = 0.f;
  for (int j = 0; j < p.k; ++j) {
    uint64_t best = 0;
    float best_s = 0.f;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const uint32_t e = (uint32_t)(s * kWave + lane);
      const uint64_t v = ((uint64_t)f32_order_key(key[s]) << 32) | (0xFFFFFFFFu - e);
      if (ok[s] && v > best) { best = v; best_s = sc[s]; }
    }
    const uint64_t w = wave_max_u64(best);
    const int id = (int)(0xFFFFFFFFu - (uint32_t)w);
    const float s_w = __shfl(best_s, id & 63, kWave);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s)
      if (s * kWave + lane == id) ok[s] = false;
    if (lane == j) { sel_id = id; sel_s = s_w; }
  }
  float wgt = sel_s;
  if (p.renorm) {
    const float sum = wave_sum(lane < p.k ? sel_s : 0.f);
    wgt = sel_s / (sum + 1e-20f);
  }
  wgt *= p.scale;
  if (lane < p.k) {
    p.ids[(size_t)t * p.k + lane] = sel_id;
    p.weights[(size_t)t * p.k + lane] = wgt;
  }
}

template <int TPB, int EPW, int SLOTS>
__global__ __launch_bounds__(256) void route_kernel(RouteParams p) {
  const int etile = blockIdx.x;
  const int ttile = blockIdx.y;
  gemv_tile<TPB, EPW>(p, ttile, etile);

  __shared__ int s_last;
  __threadfence();  // this thread's logits are visible at agent scope
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(p.counters + ttile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (unsigned)(p.n_etiles - 1);
    if (last) __hip_atomic_store(p.counters + ttile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire: see every block's logits
  const int wave = threadIdx.x >> 6;
  for (int j = wave; j < TPB; j += 4) {
    const int t = ttile * TPB + j;
    if (t < p.T) select_token<SLOTS>(p, t);
  }
}

template <int TPB, int EPW>
moe_status launch_route_tpb(const RouteParams& p0, hipStream_t stream) {
  RouteParams p = p0;
  p.n_etiles = ceil_div(p.E, 4 * EPW);
  dim3 grid(p.n_etiles, ceil_div(p.T, TPB));
  const int slots = ceil_div(p.E, kWave);
  if (slots <= 1)
    route_kernel<TPB, EPW, 1><<<grid, 256, 0, stream>>>(p);
  else if (slots <= 2)
    route_kernel<TPB, EPW, 2><<<grid, 256, 0, stream>>>(p);
  else if (slots <= 4)
    route_kernel<TPB, EPW, 4><<<grid, 256, 0, stream>>>(p);
  else if (slots <= 5)
    route_kernel<TPB, EPW, 5><<<grid, 256, 0, stream>>>(p);
  else if (slots <= 8)
    route_kernel<TPB, EPW, 8><<<grid, 256, 0, stream>>>(p);
  else
    route_kernel<TPB, EPW, 16><<<grid, 256, 0, stream>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace

size_t route_workspace_size(int T, int E) { return kCtrlBytes + align_up((size_t)T * E * sizeof(float), 256); }

static int route_tokens_per_tile(int T) { return T <= 1 ? 1 : (T <= 4 ? 4 : 16); }

moe_status route_validate(const void* x, const float* gate, int T, int H, int E, int k, int n_group,
                          int topk_group, int scoring, const int32_t* ids, const float* w) {
  if (T < 0 || H < 8 || H % 8 != 0 || E < 1 || E > 1024 || k < 1 || k > 16 || k > E) return MOE_E_INVAL;
  if (scoring != MOE_SOFTMAX && scoring != MOE_SIGMOID) return MOE_E_INVAL;
  if (n_group < 1 || n_group > 64 || E % n_group != 0) return MOE_E_INVAL;
  if (n_group > 1 && (E / n_group < 2)) return MOE_E_INVAL;
  if (topk_group < 1 || topk_group > n_group) return MOE_E_INVAL;
  if ((int64_t)k > (int64_t)topk_group * (E / n_group)) return MOE_E_INVAL;
  if (T > 0 && (!x || !gate || !ids || !w)) return MOE_E_INVAL;
  if (ceil_div(T, route_tokens_per_tile(T)) > kMaxCounters) return MOE_E_INVAL;
  return MOE_OK;
}

moe_status launch_route(const void* x, const float* gate, const float* bias, int T, int H, int E, int k,
                        int n_group, int topk_group, int scoring, int renormalize, float routed_scale,
                        int32_t* ids, float* weights, float* logits_out, void* ws, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  RouteParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.gate = gate;
  p.bias = bias;
  char* base = static_cast<char*>(ws);
  p.logits = logits_out ? logits_out : reinterpret_cast<float*>(base + kCtrlBytes);
  p.counters = reinterpret_cast<unsigned*>(base + kCounterOffset);
  p.ids = ids;
  p.weights = weights;
  p.T = T; p.H = H; p.E = E; p.k = k;
  p.n_group = n_group; p.topk_group = topk_group;
  p.scoring = scoring; p.renorm = renormalize != 0;
  p.scale = routed_scale;
  p.n_etiles = 1;
  switch (route_tokens_per_tile(T)) {
    case 1: return launch_route_tpb<1, 1>(p, stream);
    case 4: return launch_route_tpb<4, 1>(p, stream);
    default: return launch_route_tpb<16, 2>(p, stream);
  }
}

}  // namespace moe

extern "C" moe_status moe_route(const void* x, const float* gate, const float* bias, int T, int H, int E,
                                int k, int n_group, int topk_group, int scoring, int renormalize,
                                float routed_scale, int32_t* topk_ids, float* topk_weights,
                                float* logits_out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  using namespace moe;
  moe_status st = route_validate(x, gate, T, H, E, k, n_group, topk_group, scoring, topk_ids, topk_weights);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!workspace) return MOE_E_INVAL;
  if (workspace_bytes < route_workspace_size(T, E)) return MOE_E_WORKSPACE;
  return launch_route(x, gate, bias, T, H, E, k, n_group, topk_group, scoring, renormalize, routed_scale,
                      topk_ids, topk_weights, logits_out, workspace, stream);
}

extern "C" size_t moe_route_workspace_size(int T, int E) {
  if (T < 0 || E < 1) return 0;
  return moe::route_workspace_size(T, E);
}
