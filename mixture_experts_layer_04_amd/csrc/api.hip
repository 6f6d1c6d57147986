// moe_layer (route -> align -> expert FFN on one stream), status strings,
// the test-only error read-back and the measurement probes.

#include <cmath>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

struct LayerLayout {
  size_t ctrl, ids, w, sorted, bexp, npp, ffn, total;
};

// The route workspace (control block + group partials) sits at offset 0;
// the alignment workspace (the same control block + its scratch) overlaps it,
// the router being done with its partials before the alignment starts.  With
// a shared expert the ids, the alignment and the FFN cover E + 1 experts and
// k + 1 slots.
LayerLayout layer_layout(int T, int H, int E, int F, int k, int ns, int block_m, int wformat) {
  LayerLayout L;
  const int Ea = E + ns, ka = k + ns;
  size_t off = 0;
  L.ctrl = off;
  off += align_up(route_align_workspace_size(T, H, E, k, ns), 256);
  L.ids = off;
  off += align_up((size_t)T * ka * sizeof(int32_t), 256);
  L.w = off;
  off += align_up((size_t)T * ka * sizeof(float), 256);
  L.sorted = off;
  off += align_up((size_t)align_max_padded(T, ka, Ea, block_m) * sizeof(int32_t), 256);
  L.bexp = off;
  off += align_up((size_t)align_max_blocks(T, ka, Ea, block_m) * sizeof(int32_t), 256);
  L.npp = off;
  off += 256;
  L.ffn = off;
  off += align_up(ffn_workspace_size(T, H, Ea, F, ka, block_m, wformat), 256);
  L.total = off;
  return L;
}

__global__ void empty_kernel() {}

__global__ __launch_bounds__(256) void read_kernel(const uint4* p, size_t n16, float* sink) {
  float acc = 0.f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
    const uint4 v = p[i];
    acc += __uint_as_float(v.x ^ v.y ^ v.z ^ v.w);
  }
  acc = wave_sum(acc);
  __shared__ float s[4];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] + s[1] + s[2] + s[3];
}

int read_grid(size_t bytes) {
  const size_t n16 = bytes / 16;
  size_t g = (n16 + 255) / 256;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

// Block size for T tokens.  Below 2 rows per expert on average most blocks
// hold one or two rows; the 16-row weight-stream kernel spreads the weights
// of the few experts touched over every CU, while the 32-row tiled kernel
// needs enough tiles to fill them: one per (expert touched, 256 GEMM1
// weight rows), with E (1 - (1 - k/E)^T) experts touched.  Measured (cold
// layers): bf16 turns to the tiled kernel at about 400 such tiles, MX (whose
// 32-row kernel takes 256-wide K steps) at about 320, and fp8 keeps the
// stream kernel up to 2 rows per expert.  From 2 rows on, the smallest
// block that the expected rows per expert fill, with the cuts measured on
// the tiled kernels.
int layer_block_m(int T, int k, int E, int F, int wformat) {
  const double m = (double)T * k / E;  // rows per expert
  if (m < 2.0) {
    if (wformat == MOE_W_FP8_BLOCK128) return 16;
    const double touched = E * (1.0 - std::pow(1.0 - (double)k / E, (double)T));
    const double tiles = touched * (2.0 * F / 256.0);
    return tiles >= (wformat == MOE_W_MXFP4 ? 320.0 : 400.0) ? 32 : 16;
  }
  if (m <= 24.0) return 32;
  // fp8 (the tiled kernel, which copies an expert's weight tile once per
  // block and skips the fragments of padding rows): 128 rows from m = 48 on
  // (measured, DSV3 layers, 64 against 128 rows: m = 32 2148 / 2186 us,
  // m = 40 2212 / 2237, m = 48 2357 / 2272, m = 64 2670 / 2374)
  if (wformat == MOE_W_FP8_BLOCK128) return m <= 44.0 ? 64 : 128;
  if (m <= 96.0) return 64;
  return 128;
}

}  // namespace moe

#ifndef MOE_SOURCE_HASH
#define MOE_SOURCE_HASH "unknown"
#endif
extern "C" const char* moe_source_hash(void) { return MOE_SOURCE_HASH; }

extern "C" const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_INVAL: return "MOE_E_INVAL: invalid argument";
    case MOE_E_UNSUPPORTED: return "MOE_E_UNSUPPORTED: unsupported shape or format";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace too small";
    case MOE_E_HIP: return "MOE_E_HIP: HIP runtime error at launch";
  }
  return "unknown moe_status";
}

extern "C" int moe_layer_block_m(int T, int E, int F, int k, int wformat) {
  if (T < 0 || k < 1 || E < 1 || F < 1) return 16;
  return moe::layer_block_m(T, k, E, F, wformat);
}

namespace moe {
size_t layer_workspace_bytes(int T, int H, int E, int F, int k, int n_shared, int block_m, int wformat) {
  if (T < 0 || H < 1 || E < 1 || F < 1 || k < 1 || n_shared < 0 || n_shared > 1) return 0;
  if (block_m == 0) block_m = layer_block_m(T, k + n_shared, E + n_shared, F, wformat);
  return layer_layout(T, H, E, F, k, n_shared, block_m, wformat).total;
}
}  // namespace moe

extern "C" size_t moe_layer_workspace_size(int T, int H, int E, int F, int k, int n_shared, int block_m,
                                           int wformat) {
  return moe::layer_workspace_bytes(T, H, E, F, k, n_shared, block_m, wformat);
}

namespace moe {

moe_status layer_validate(const void* x, const void* gate, int gate_is_fp32, int wformat, const void* w13,
                          const void* w13_scale,
                          const void* w2, const void* w2_scale, int T, int H, int E, int F, int k, int n_shared,
                          int n_group, int topk_group, int scoring, int block_m, float swiglu_limit, const void* y) {
  if (n_shared != 0 && n_shared != 1) return MOE_E_INVAL;
  const int Ea = E + n_shared, ka = k + n_shared;
  if (block_m == 0) block_m = (T >= 0 && k >= 1 && E >= 1 && F >= 1) ? layer_block_m(T, ka, Ea, F, wformat) : 16;
  int32_t dummy_i = 0;
  float dummy_f = 0.f;
  moe_status st = route_validate(x, gate, gate_is_fp32, T, H, E, k, n_group, topk_group, scoring, &dummy_i, &dummy_f);
  if (st != MOE_OK) return st;
  return ffn_validate(x, wformat, w13, w13_scale, w2, w2_scale, &dummy_i, &dummy_f, &dummy_i, &dummy_i, &dummy_i,
                      T, H, Ea, F, ka, block_m, swiglu_limit, y);
}

moe_status layer_enqueue(const void* x, const void* gate, int gate_is_fp32, const float* bias, int wformat,
                         const void* w13,
                         const void* w13_scale, const void* w2, const void* w2_scale, int T, int H, int E, int F,
                         int k, int n_shared, int n_group, int topk_group, int scoring, int renormalize,
                         float routed_scale, int block_m, float swiglu_limit, void* y, int32_t* topk_ids_out,
                         float* topk_weights_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // validate everything before enqueuing anything
  moe_status st = layer_validate(x, gate, gate_is_fp32, wformat, w13, w13_scale, w2, w2_scale, T, H, E, F, k,
                                 n_shared, n_group, topk_group, scoring, block_m, swiglu_limit, y);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const int Ea = E + n_shared, ka = k + n_shared;  // the expert FFN sees the shared expert as expert E
  if (block_m == 0) block_m = layer_block_m(T, ka, Ea, F, wformat);
  if (!workspace) return MOE_E_INVAL;
  const LayerLayout L = layer_layout(T, H, E, F, k, n_shared, block_m, wformat);
  if (workspace_bytes < L.total) return MOE_E_WORKSPACE;
  char* b = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(b + L.ids);
  float* w = topk_weights_out ? topk_weights_out : reinterpret_cast<float*>(b + L.w);
  int32_t* sorted = reinterpret_cast<int32_t*>(b + L.sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(b + L.bexp);
  int32_t* npp = reinterpret_cast<int32_t*>(b + L.npp);

  FfnArgs a;
  a.x = x; a.wformat = wformat;
  a.w13 = w13; a.w13_scale = w13_scale; a.w2 = w2; a.w2_scale = w2_scale;
  a.topk_ids = ids; a.topk_weights = w;
  a.sorted_ids = sorted; a.block_expert = bexp; a.num_post_padded = npp;
  a.T = T; a.H = H; a.E = Ea; a.F = F; a.k = ka; a.block_m = block_m;
  a.swiglu_limit = swiglu_limit;
  a.stages = MOE_STAGE_ALL;
  a.y = y;
  a.ctrl = b + L.ctrl;  // the FFN's own region moves with the shapes; counters stay here
  ffn_carve(a, b + L.ffn);
  // at decode the router quantises x for the fp8 formats on the way (one
  // launch fewer)
  const int qfmt = wformat == MOE_W_FP8_BLOCK128 ? 1 : wformat == MOE_W_MXFP4 ? 2 : 0;
  a.x_ready = qfmt != 0 && route_quantizes_x(T, E, H);
  // the alignment also writes the paired tiles' pair table where it can
  // (one launch fewer); the FFN builds it otherwise
  bool pairs_written = false;
  st = launch_route_align(x, gate, gate_is_fp32, bias, T, H, E, k, n_group, topk_group, scoring, renormalize,
                          routed_scale,
                          n_shared, block_m, ids, w, sorted, bexp, npp, b + L.ctrl, stream, a.xq, a.xs, qfmt,
                          static_cast<int32_t*>(a.pairs), &pairs_written, /*fill_tail=*/false);
  if (st != MOE_OK) return st;
  a.pairs_ready = pairs_written;
  return launch_ffn(a, stream);
}

}  // namespace moe

extern "C" moe_status moe_layer(const void* x, const void* gate, int gate_is_fp32, const float* bias, int wformat,
                                const void* w13, const void* w13_scale, const void* w2, const void* w2_scale,
                                int T, int H, int E, int F, int k, int n_shared, int n_group, int topk_group,
                                int scoring, int renormalize, float routed_scale, int block_m, float swiglu_limit,
                                void* y, int32_t* topk_ids_out, float* topk_weights_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return moe::layer_enqueue(x, gate, gate_is_fp32, bias, wformat, w13, w13_scale, w2, w2_scale, T, H, E, F, k,
                            n_shared, n_group,
                            topk_group, scoring, renormalize, routed_scale, block_m, swiglu_limit, y, topk_ids_out,
                            topk_weights_out, workspace, workspace_bytes, stream);
}

extern "C" int32_t moe_debug_error(void* workspace, hipStream_t stream) {
  int32_t v = 0;
  if (!workspace) return -1;
  if (hipStreamSynchronize(stream) != hipSuccess) return -1;
  if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return -1;
  const int32_t zero = 0;
  if (hipMemcpy(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return -1;
  return v;
}

extern "C" moe_status moe_probe_empty(hipStream_t stream) {
  moe::empty_kernel<<<1, 64, 0, stream>>>();
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" size_t moe_probe_read_sink_len(size_t bytes) { return (size_t)moe::read_grid(bytes); }

extern "C" moe_status moe_probe_read(const void* p, size_t bytes, float* sink, hipStream_t stream) {
  if (!p || !sink || bytes == 0 || bytes % 16) return MOE_E_INVAL;
  const int g = moe::read_grid(bytes);
  moe::read_kernel<<<g, 256, 0, stream>>>(static_cast<const uint4*>(p), bytes / 16, sink);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
