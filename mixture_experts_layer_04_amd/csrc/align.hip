// Block alignment in one launch of one workgroup.
//
// [MoE] "vLLM's Triton path: align, then index" (per-expert counts, each
// rounded up to a whole block, exclusive scan, block-to-expert table, -1
// after the padded length) and [Kernels] "Alignment: making ragged routing
// tileable" (flat assignment ids, sentinel T*k, worst-case sizing
// T*k + E*(BLOCK_M-1) so the padded length can stay on the device).
//
// Unlike an atomic-add placement, every position here is decided without
// atomics, so the layout is deterministic and stable (ascending assignment id
// within an expert):
//   1. each wave owns one contiguous segment of the assignments and counts its
//      ids per expert into its own LDS row cnt[w][e];
//   2. counts are summed over waves, padded to a multiple of BLOCK_M and
//      scanned (wave 0); cnt[w][e] becomes wave w's first slot for expert e;
//   3. each wave walks its segment again 64 assignments at a time; lanes with
//      equal ids find each other with one ballot per id bit, take
//      rank = #equal lanes below them, and the lowest such lane advances
//      cnt[w][e] by the group size.
// Padding slots and the tail get the sentinel T*k; block_expert is filled by
// a binary search of the scanned starts and -1 past the padded length.

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

struct AlignParams {
  const int32_t* ids;
  int32_t* sorted_ids;
  int32_t* block_expert;
  int32_t* num_post_padded;
  int32_t* err;
  int A, E, bm, nbits;
  int max_padded, max_blocks;
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void align_kernel(AlignParams p) {
  extern __shared__ int smem[];
  int* cnt = smem;                   // [NW][E]
  int* start = smem + NW * p.E;      // [E + 1]
  int* count = start + p.E + 1;      // [E]
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int NT = NW * 64;
  const int A = p.A;
  const int E = p.E;

  // segment of this wave, a multiple of 64 long
  const int seg = ((A + NW - 1) / NW + 63) & ~63;
  const int a_begin = min(A, wave * seg);
  const int a_end = min(A, a_begin + seg);

  int* my = cnt + wave * E;
  for (int e = lane; e < E; e += 64) my[e] = 0;
  bool bad = false;
  // ids are read CH per lane at a time (all loads in flight together)
  constexpr int CH = 16;
  for (int a0 = a_begin; a0 < a_end; a0 += 64 * CH) {
    int idv[CH];
    const int nc = min(CH, (a_end - a0 + 63) >> 6);  // sub-chunks of 64 holding ids
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int a = a0 + 64 * c + lane;
      idv[c] = (c < nc && a < a_end) ? p.ids[a] : -1;
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c >= nc) break;
      const int id = idv[c];
      if (id >= 0 && id < E)
        atomicAdd(&my[id], 1);
      else if (id != -1)
        bad = true;
    }
  }
  if (__ballot(bad) != 0ull && lane == 0) atomicOr(p.err, 1);
  __syncthreads();

  // per-expert totals and padded sizes
  for (int e = tid; e < E; e += NT) {
    int c = 0;
    for (int w = 0; w < NW; ++w) c += cnt[w * E + e];
    count[e] = c;
    start[e] = (c + p.bm - 1) / p.bm * p.bm;  // padded, scanned below
  }
  __syncthreads();

  // exclusive scan of the padded sizes by wave 0 (each lane a run of E/64)
  if (wave == 0) {
    const int per = (E + 63) / 64;
    const int lo = min(E, lane * per);
    const int hi = min(E, lo + per);
    int run = 0;
    for (int e = lo; e < hi; ++e) run += start[e];
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int excl = incl - run;
    for (int e = lo; e < hi; ++e) {
      const int v = start[e];
      start[e] = excl;
      excl += v;
    }
    if (lane == 63) start[E] = incl;
  }
  __syncthreads();

  const int total = start[E];
  if (tid == 0) p.num_post_padded[0] = total;
  // first slot of each (wave, expert)
  for (int e = tid; e < E; e += NT) {
    int run = start[e];
    for (int w = 0; w < NW; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
  }
  // sentinel in the padding of each expert and in the tail
  for (int e = tid; e < E; e += NT)
    for (int i = start[e] + count[e]; i < start[e + 1]; ++i) p.sorted_ids[i] = A;
  for (int i = total + tid; i < p.max_padded; i += NT) p.sorted_ids[i] = A;
  // block table
  const int nb = total / p.bm;
  for (int b = tid; b < p.max_blocks; b += NT) {
    int e = -1;
    if (b < nb) {
      const int row = b * p.bm;
      int lo = 0, hi = E + 1;  // upper_bound of row in start[0..E]
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (start[mid] <= row) lo = mid + 1; else hi = mid;
      }
      e = lo - 1;
    }
    p.block_expert[b] = e;
  }
  __syncthreads();

  // stable placement
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int a1 = a_begin; a1 < a_end; a1 += 64 * CH) {
    int idv[CH];
    const int nc = min(CH, (a_end - a1 + 63) >> 6);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int a = a1 + 64 * c + lane;
      idv[c] = (c < nc && a < a_end) ? p.ids[a] : -1;
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {  // 64 consecutive assignments at a time, in order
      if (c >= nc) break;
      const int a = a1 + 64 * c + lane;
      int id = idv[c];
      const bool valid = id >= 0 && id < E;
      if (!valid) id = 0;
      uint64_t m = __ballot(valid);
      for (int b = 0; b < p.nbits; ++b) {
        const bool bit = (id >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      if (valid) {
        const int rank = __popcll(m & lt);
        const int pos = my[id] + rank;
        p.sorted_ids[pos] = a;
        if (rank == 0) my[id] += __popcll(m);
      }
    }
  }
}

}  // namespace

int align_waves(int E) { return E <= 512 ? 16 : 8; }

size_t align_lds_bytes(int E) { return ((size_t)align_waves(E) * E + 2 * E + 1) * sizeof(int); }

moe_status align_validate(const int32_t* ids, int T, int k, int E, int block_m, const void* sorted_ids,
                          const void* block_expert, const void* num_post_padded) {
  if (T < 0 || k < 1 || k > 16 || E < 1 || E > 1024) return MOE_E_INVAL;
  if (block_m < 1 || block_m > 1024) return MOE_E_INVAL;
  if ((int64_t)T * k > (1 << 24)) return MOE_E_INVAL;
  if (!sorted_ids || !block_expert || !num_post_padded) return MOE_E_INVAL;
  if (T > 0 && !ids) return MOE_E_INVAL;
  return MOE_OK;
}

moe_status launch_align(const int32_t* ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_post_padded, void* ws, hipStream_t stream) {
  AlignParams p;
  p.ids = ids;
  p.sorted_ids = sorted_ids;
  p.block_expert = block_expert;
  p.num_post_padded = num_post_padded;
  p.err = static_cast<int32_t*>(ws);
  p.A = T * k;
  p.E = E;
  p.bm = block_m;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  p.nbits = nbits;
  p.max_padded = (int)align_max_padded(T, k, E, block_m);
  p.max_blocks = (int)align_max_blocks(T, k, E, block_m);
  const size_t lds = align_lds_bytes(E);
  if (align_waves(E) == 16)
    align_kernel<16><<<1, 16 * 64, lds, stream>>>(p);
  else
    align_kernel<8><<<1, 8 * 64, lds, stream>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

int64_t align_max_padded(int T, int k, int E, int block_m) {
  return (int64_t)T * k + (int64_t)E * (block_m - 1);
}
int64_t align_max_blocks(int T, int k, int E, int block_m) {
  return ceil_div64(align_max_padded(T, k, E, block_m), block_m);
}
size_t align_workspace_size() { return kCtrlBytes; }

}  // namespace moe

extern "C" moe_status moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m,
                                int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_padded,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace moe;
  moe_status st = align_validate(topk_ids, T, k, E, block_m, sorted_ids, block_expert, num_post_padded);
  if (st != MOE_OK) return st;
  if (!workspace) return MOE_E_INVAL;
  if (workspace_bytes < align_workspace_size()) return MOE_E_WORKSPACE;
  return launch_align(topk_ids, T, k, E, block_m, sorted_ids, block_expert, num_post_padded, workspace,
                      stream);
}

extern "C" size_t moe_align_workspace_size(int T, int k, int E) {
  (void)T; (void)k; (void)E;
  return moe::align_workspace_size();
}
extern "C" int64_t moe_align_max_padded(int T, int k, int E, int block_m) {
  return moe::align_max_padded(T, k, E, block_m);
}
extern "C" int64_t moe_align_max_blocks(int T, int k, int E, int block_m) {
  return moe::align_max_blocks(T, k, E, block_m);
}
