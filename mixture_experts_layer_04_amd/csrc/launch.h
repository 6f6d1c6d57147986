// Internal (host-side) launchers shared between the entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Every workspace starts with a fixed control block that no other region of
// any entry point overlaps, so whatever sequence of shapes shares one
// workspace, the words in it only ever hold what their owners leave there
// (zero after each call):
//   [0, 4)            sticky alignment error bits
//   [4, 8)            alignment counter (multi-workgroup path)
//   [16, 52)          grouped GEMM tile queues: one per XCD, then the
//                     count of workgroups done
//   [256, kCtrlBytes) one counter per router token tile
constexpr size_t kCtrlBytes = 65536;
constexpr size_t kAlignCounterOffset = 4;
constexpr size_t kTileQueueOffset = 16;
constexpr size_t kCounterOffset = 256;
constexpr int kMaxCounters = (int)((kCtrlBytes - kCounterOffset) / 4);

moe_status route_validate(const void* x, const void* gate, int gate_is_fp32, int T, int H, int E, int k, int n_group,
                          int topk_group, int scoring, const int32_t* ids, const float* w);
size_t route_workspace_size(int T, int H, int E);
moe_status launch_route(const void* x, const void* gate, int gate_is_fp32, const float* bias, int T, int H, int E,
                        int k,
                        int n_group, int topk_group, int scoring, int renormalize, float routed_scale,
                        int32_t* ids, float* weights, float* logits_out, void* ws, hipStream_t stream);

// Route + align in one call: one launch while T <= 4 (the router's decode
// layout, whose last token tile aligns every assignment), else the router's
// two launches and launch_align.
// n_shared = 1: slot k of every token is the shared expert (id E, weight 1),
// ids / weights rows hold k + 1 slots and the alignment covers E + 1 experts.
// qfmt 1 (FP8) / 2 (MX): where route_quantizes_x(T, E, H), the router also
// quantises x into xq / xs as the FFN's activation stage would; 0: no.
moe_status launch_route_align(const void* x, const void* gate, int gate_is_fp32, const float* bias, int T, int H,
                              int E, int k,
                              int n_group, int topk_group, int scoring, int renormalize, float routed_scale,
                              int n_shared, int block_m, int32_t* ids, float* weights, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* num_post_padded, void* ws, hipStream_t stream,
                              void* xq, void* xs, int qfmt, int32_t* pairs = nullptr,
                              bool* pairs_written = nullptr, bool fill_tail = true);
bool route_quantizes_x(int T, int E, int H);
size_t route_align_workspace_size(int T, int H, int E, int k, int n_shared);

moe_status align_validate(const int32_t* ids, int T, int k, int E, int block_m, const void* sorted_ids,
                          const void* block_expert, const void* num_post_padded);
size_t align_workspace_size(int T, int k, int E);
int64_t align_max_padded(int T, int k, int E, int block_m);
int64_t align_max_blocks(int T, int k, int E, int block_m);
// pairs (optional): also write the paired GEMM tiles' pair table there
// (*pairs_written says whether it did: not for at most 64 assignments)
moe_status launch_align(const int32_t* ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_post_padded, void* ws, hipStream_t stream,
                        int32_t* pairs = nullptr, bool* pairs_written = nullptr, bool fill_tail = true);

// Everything moe_expert_ffn needs, with the workspace already carved.
struct FfnArgs {
  const void* x;
  int wformat;
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
  const int32_t* topk_ids;
  const float* topk_weights;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* num_post_padded;
  int T, H, E, F, k, block_m;
  float swiglu_limit;  // +inf: no clamp
  int stages;      // bit mask of MOE_STAGE_* to run
  bool x_ready;    // xq / xs already hold the quantised x (the router wrote them)
  bool pairs_ready;  // the pair table was written by the alignment (launch_align's pairs)
  void* y;
  // workspace regions
  void* xq;        // quantised x (fp8 formats)
  void* xs;        // its scales
  void* act;       // SwiGLU output [max_padded, F]
  void* act_s;     // its scales (fp8 formats)
  void* act32;     // BLOCK_M 16 with fp8 formats: fp32 SwiGLU rows before requantisation
  void* out;       // expert outputs [T*k, H] bf16
  void* pairs;     // paired tiled GEMMs (ffn_paired): pair table, max_blocks + 1 ints; else null
  void* ctrl;      // control block of the caller's workspace (tile queues)
};

moe_status ffn_validate(const void* x, int wformat, const void* w13, const void* w13_scale, const void* w2,
                        const void* w2_scale, const int32_t* topk_ids, const float* topk_weights,
                        const int32_t* sorted_ids, const int32_t* block_expert,
                        const int32_t* num_post_padded, int T, int H, int E, int F, int k, int block_m,
                        float swiglu_limit, const void* y);
size_t ffn_workspace_size(int T, int H, int E, int F, int k, int block_m, int wformat);
// Whether the grouped GEMMs run the paired tiled kernel (two blocks of one
// expert per tile), which needs the pair table built first.
bool ffn_paired(int wformat, int block_m, int T, int k, int E);
moe_status launch_pair_table(const FfnArgs& a, hipStream_t stream);
void ffn_carve(FfnArgs& a, void* ws);
moe_status launch_ffn(const FfnArgs& a, hipStream_t stream);

// per-format GEMM launchers; `which` is 1 for GEMM1 (+SwiGLU), 2 for GEMM2
moe_status launch_gemm_bf16(const FfnArgs& a, int which, hipStream_t stream);
moe_status launch_gemm_fp8(const FfnArgs& a, int which, hipStream_t stream);
moe_status launch_gemm_mxfp4(const FfnArgs& a, int which, hipStream_t stream);
moe_status launch_quant_x(const FfnArgs& a, hipStream_t stream);
moe_status launch_finalize(const FfnArgs& a, hipStream_t stream);

// Grid size for a grid-stride loop over `n_tiles` tiles that are spread over
// the 8 XCDs in contiguous runs (see xcd_tile()).
int tile_grid(int64_t n_tiles, int max_wgs);

// moe_layer's checks (scalars, formats, non-null pointers), and moe_layer on
// a caller-chosen workspace (checks first, then route + align + expert FFN).
size_t layer_workspace_bytes(int T, int H, int E, int F, int k, int n_shared, int block_m, int wformat);
moe_status layer_validate(const void* x, const void* gate, int gate_is_fp32, int wformat, const void* w13,
                          const void* w13_scale,
                          const void* w2, const void* w2_scale, int T, int H, int E, int F, int k, int n_shared,
                          int n_group, int topk_group, int scoring, int block_m, float swiglu_limit, const void* y);
moe_status layer_enqueue(const void* x, const void* gate, int gate_is_fp32, const float* bias, int wformat,
                         const void* w13,
                         const void* w13_scale, const void* w2, const void* w2_scale, int T, int H, int E, int F,
                         int k, int n_shared, int n_group, int topk_group, int scoring, int renormalize,
                         float routed_scale, int block_m, float swiglu_limit, void* y, int32_t* topk_ids_out,
                         float* topk_weights_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

}  // namespace moe

#ifdef __HIPCC__
namespace moe {
// Maps the i-th grid-stride tile index to a logical tile so that XCD x
// (workgroups are dealt to the XCDs round-robin) handles the contiguous run
// [x*per, (x+1)*per) of logical tiles: neighbouring logical tiles (the N
// tiles of one block) share their A rows in that XCD's L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t i, int64_t per) { return (i & 7) * per + (i >> 3); }
}  // namespace moe
#endif
