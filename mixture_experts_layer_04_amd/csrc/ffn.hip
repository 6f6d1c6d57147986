// moe_expert_ffn: argument checks, workspace layout, the combine kernel and
// the per-format dispatch.
//
// Combine ([Kernels] "Combine, backward and low precision": a gather per
// token that sums its k rows in a fixed order is deterministic; [MegaMoE]
// §3.7: the slots of a token are added as fp32 in slot order and rounded
// once): one workgroup per token reads the token's k expert-output rows,
// multiplies each by its routing weight and adds them in slot order in fp32.

#include "combine.h"
#include "common.h"
#include "launch.h"

namespace moe {

int tile_grid(int64_t n_tiles, int max_wgs) {
  int64_t g = n_tiles < max_wgs ? n_tiles : max_wgs;
  g = (g + 7) / 8 * 8;
  return (int)(g < 8 ? 8 : g);
}

namespace {

struct FinP {
  const uint16_t* out;
  const int32_t* ids;
  const float* w;
  uint16_t* y;
  int H, E, k;
};

// grid (T, column splits): a workgroup takes every gridDim.y-th run of 2048
// columns of token blockIdx.x (at small T the columns of a token are split
// over several workgroups, so each thread makes one pass)
template <int KT>  // = k
__global__ __launch_bounds__(256) void finalize_kernel(FinP p) {
  const int t = blockIdx.x;
  const int32_t* ids = p.ids + (size_t)t * p.k;
  const float* w = p.w + (size_t)t * p.k;
  for (int h = (blockIdx.y * 256 + threadIdx.x) * 8; h < p.H; h += gridDim.y * 256 * 8)
    *reinterpret_cast<uint4*>(p.y + (size_t)t * p.H + h) = combine8<KT>(p.out, ids, w, t, h, p.H, p.E, KT);
}

}  // namespace

moe_status launch_finalize(const FfnArgs& a, hipStream_t s) {
  FinP p;
  p.out = static_cast<const uint16_t*>(a.out);
  p.ids = a.topk_ids;
  p.w = a.topk_weights;
  p.y = static_cast<uint16_t*>(a.y);
  p.H = a.H; p.E = a.E; p.k = a.k;
  const dim3 grid(a.T, a.T < 512 ? (a.H + 2047) / 2048 : 1);
  switch (a.k) {
#define MOE_FIN(K) \
  case K: finalize_kernel<K><<<grid, 256, 0, s>>>(p); break;
    MOE_FIN(1) MOE_FIN(2) MOE_FIN(3) MOE_FIN(4) MOE_FIN(5) MOE_FIN(6) MOE_FIN(7) MOE_FIN(8)
    MOE_FIN(9) MOE_FIN(10) MOE_FIN(11) MOE_FIN(12) MOE_FIN(13) MOE_FIN(14) MOE_FIN(15) MOE_FIN(16)
#undef MOE_FIN
    default: return MOE_E_INVAL;
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

moe_status ffn_validate(const void* x, int wformat, const void* w13, const void* w13_scale, const void* w2,
                        const void* w2_scale, const int32_t* topk_ids, const float* topk_weights,
                        const int32_t* sorted_ids, const int32_t* block_expert,
                        const int32_t* num_post_padded, int T, int H, int E, int F, int k, int block_m,
                        float swiglu_limit, const void* y) {
  if (T < 0 || H < 128 || F < 128 || H % 128 || F % 128) return MOE_E_INVAL;
  if (!(swiglu_limit > 0.f)) return MOE_E_INVAL;  // NaN or <= 0
  if (E < 1 || E > 1024 || k < 1 || k > 16 || k > E) return MOE_E_INVAL;
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128) return MOE_E_INVAL;
  if ((int64_t)T * k > (1 << 24)) return MOE_E_INVAL;
  if (wformat != MOE_W_BF16 && wformat != MOE_W_FP8_BLOCK128 && wformat != MOE_W_MXFP4) return MOE_E_INVAL;
  if (T == 0) return MOE_OK;
  if (!x || !w13 || !w2 || !topk_ids || !topk_weights || !sorted_ids || !block_expert || !num_post_padded || !y)
    return MOE_E_INVAL;
  if (wformat != MOE_W_BF16 && (!w13_scale || !w2_scale)) return MOE_E_INVAL;
  if (wformat != MOE_W_BF16 && (H % 512 != 0 || F % 512 != 0)) return MOE_E_UNSUPPORTED;
  // x, the SwiGLU rows and one expert's weights are addressed with 32-bit
  // byte offsets
  const uint64_t eb = wformat == MOE_W_BF16 ? 2 : 1, lim = 0xFFFFFFFFull;
  if ((uint64_t)T * H * eb > lim || (uint64_t)align_max_padded(T, k, E, block_m) * F * eb > lim ||
      (uint64_t)2 * F * H * eb > lim)
    return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

namespace {
struct Layout {
  size_t xq, xs, act, act_s, act32, out, pairs, total;
};
Layout ffn_layout(int T, int H, int E, int F, int k, int block_m, int wformat) {
  Layout L;
  const size_t mp = (size_t)align_max_padded(T, k, E, block_m);
  size_t off = 0;
  const bool q = wformat != MOE_W_BF16;
  off += kCtrlBytes;  // never written by the FFN; keeps the control block intact
  L.xq = off;
  off += q ? align_up((size_t)T * H, 256) : 0;
  L.xs = off;
  off += q ? align_up((size_t)T * (H / 32) * sizeof(float), 256) : 0;
  L.act = off;
  off += align_up(mp * F * (q ? 1 : 2), 256);
  L.act_s = off;
  off += q ? align_up(mp * (F / 32) * sizeof(float), 256) : 0;
  L.act32 = off;
  off += (q && block_m == 16) ? align_up(mp * F * sizeof(float), 256) : 0;
  L.out = off;
  off += align_up((size_t)T * k * H * 2, 256);
  L.pairs = off;
  off += ffn_paired(wformat, block_m, T, k, E) ? align_up(((size_t)align_max_blocks(T, k, E, block_m) + 1) * 4, 256)
                                                : 0;
  L.total = off;
  return L;
}
}  // namespace

size_t ffn_workspace_size(int T, int H, int E, int F, int k, int block_m, int wformat) {
  return ffn_layout(T, H, E, F, k, block_m, wformat).total;
}

void ffn_carve(FfnArgs& a, void* ws) {
  const Layout L = ffn_layout(a.T, a.H, a.E, a.F, a.k, a.block_m, a.wformat);
  char* b = static_cast<char*>(ws);
  a.xq = b + L.xq;
  a.xs = b + L.xs;
  a.act = b + L.act;
  a.act_s = b + L.act_s;
  a.act32 = b + L.act32;
  a.out = b + L.out;
  a.pairs = ffn_paired(a.wformat, a.block_m, a.T, a.k, a.E) ? b + L.pairs : nullptr;
}

static moe_status launch_gemm(const FfnArgs& a, int which, hipStream_t s) {
  switch (a.wformat) {
    case MOE_W_BF16: return launch_gemm_bf16(a, which, s);
    case MOE_W_FP8_BLOCK128: return launch_gemm_fp8(a, which, s);
    case MOE_W_MXFP4: return launch_gemm_mxfp4(a, which, s);
  }
  return MOE_E_INVAL;
}

moe_status launch_ffn(const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return MOE_OK;
  moe_status st = MOE_OK;
  if ((a.stages & MOE_STAGE_QUANT) && a.wformat != MOE_W_BF16 && !a.x_ready) st = launch_quant_x(a, s);
  if (st == MOE_OK && a.pairs && !a.pairs_ready && (a.stages & MOE_STAGE_QUANT)) st = launch_pair_table(a, s);
  if (st == MOE_OK && (a.stages & MOE_STAGE_GEMM1)) st = launch_gemm(a, 1, s);
  if (st == MOE_OK && (a.stages & MOE_STAGE_GEMM2)) st = launch_gemm(a, 2, s);
  if (st == MOE_OK && (a.stages & MOE_STAGE_COMBINE)) st = launch_finalize(a, s);
  return st;
}

}  // namespace moe

extern "C" moe_status moe_expert_ffn_stages(const void* x, int wformat, const void* w13, const void* w13_scale,
                                            const void* w2, const void* w2_scale, const int32_t* topk_ids,
                                            const float* topk_weights, const int32_t* sorted_ids,
                                            const int32_t* block_expert, const int32_t* num_post_padded,
                                            int T, int H, int E, int F, int k, int block_m,
                                            float swiglu_limit, void* y, void* workspace,
                                            size_t workspace_bytes, int stages, hipStream_t stream) {
  using namespace moe;
  if (stages & ~MOE_STAGE_ALL) return MOE_E_INVAL;
  moe_status st = ffn_validate(x, wformat, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids,
                               block_expert, num_post_padded, T, H, E, F, k, block_m, swiglu_limit, y);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!workspace) return MOE_E_INVAL;
  if (workspace_bytes < ffn_workspace_size(T, H, E, F, k, block_m, wformat)) return MOE_E_WORKSPACE;
  FfnArgs a;
  a.x = x; a.wformat = wformat;
  a.w13 = w13; a.w13_scale = w13_scale; a.w2 = w2; a.w2_scale = w2_scale;
  a.topk_ids = topk_ids; a.topk_weights = topk_weights;
  a.sorted_ids = sorted_ids; a.block_expert = block_expert; a.num_post_padded = num_post_padded;
  a.T = T; a.H = H; a.E = E; a.F = F; a.k = k; a.block_m = block_m;
  a.swiglu_limit = swiglu_limit;
  a.stages = stages;
  a.x_ready = false;
  a.pairs_ready = false;
  a.y = y;
  a.ctrl = workspace;
  ffn_carve(a, workspace);
  return launch_ffn(a, stream);
}

extern "C" moe_status moe_expert_ffn(const void* x, int wformat, const void* w13, const void* w13_scale,
                                     const void* w2, const void* w2_scale, const int32_t* topk_ids,
                                     const float* topk_weights, const int32_t* sorted_ids,
                                     const int32_t* block_expert, const int32_t* num_post_padded, int T,
                                     int H, int E, int F, int k, int block_m, float swiglu_limit, void* y,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return moe_expert_ffn_stages(x, wformat, w13, w13_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids,
                               block_expert, num_post_padded, T, H, E, F, k, block_m, swiglu_limit, y, workspace,
                               workspace_bytes, MOE_STAGE_ALL, stream);
}

extern "C" size_t moe_expert_ffn_workspace_size(int T, int H, int E, int F, int k, int block_m, int wformat) {
  if (T < 0 || H < 1 || E < 1 || F < 1 || k < 1) return 0;
  return moe::ffn_workspace_size(T, H, E, F, k, block_m, wformat);
}
