// Block alignment: one launch of one workgroup for small T*k (the device
// code in align_block.h, which the router's fused launch shares), two
// multi-workgroup launches (count, place) for large T*k.
//
// [MoE] "vLLM's Triton path: align, then index" (per-expert counts, each
// rounded up to a whole block, exclusive scan, block-to-expert table, -1
// after the padded length) and [Kernels] "Alignment: making ragged routing
// tileable" (flat assignment ids, sentinel T*k, worst-case sizing
// T*k + E*(BLOCK_M-1) so the padded length can stay on the device).
//
// Unlike an atomic-add placement, every position is decided without atomics,
// so the layout is deterministic and stable (ascending assignment id within
// an expert).  For large T*k the steps are spread over G workgroups,
// workgroup g owning the contiguous chunk [g*C, (g+1)*C) of assignments:
//   count: each workgroup writes its per-expert counts cnt[e][g]; the last
//          one to finish (agent-scope counter) sums, pads and scans them and
//          turns cnt[e][g] into workgroup g's first slot for expert e;
//          The count launch also fills every slot with the sentinel;
//   place: each workgroup recounts its chunk per wave, offsets the waves
//          from cnt[e][g] and places as the one-workgroup kernel does; all
//          workgroups share the block table.
// Positions are the same as in the one-workgroup kernel.

#include "align_block.h"
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

template <int NW>
__global__ __launch_bounds__(NW * 64) void align_kernel(AlignParams p) {
  extern __shared__ int smem[];
  if (p.A <= 64)
    align_tiny<NW>(p);
  else
    align_block<NW>(p, smem);
}

// ---------------------------------------------------------------------------
// Multi-workgroup path.
struct Align2Params {
  const int32_t* ids;
  int32_t* sorted_ids;
  int32_t* block_expert;
  int32_t* num_post_padded;
  int32_t* err;
  unsigned* counter;  // control-block word, zero between calls
  int32_t* cnt;       // [E][G] counts, then first slots
  int32_t* start;     // [E + 1] scanned padded sizes
  int32_t* pairs;     // optional pair table (write_pair_table), written by the last counting workgroup
  int A, E, bm, nbits, C, G, max_padded, max_blocks;
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void align_count_kernel(Align2Params p) {
  extern __shared__ int smem[];
  int* h = smem;              // [E] this workgroup's counts; last workgroup: padded sizes
  int* st = smem + p.E;       // [E + 1] (last workgroup)
  int* M = st + p.E + 1;      // [E][G] every workgroup's counts (last workgroup)
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NT = NW * 64;
  const int E = p.E;
  for (int e = tid; e < E; e += NT) h[e] = 0;
  for (int i = blockIdx.x * NT + tid; i < p.max_padded; i += p.G * NT) p.sorted_ids[i] = p.A;
  __syncthreads();
  const int g = blockIdx.x;
  const int c0 = g * p.C, c1 = min(p.A, c0 + p.C);
  const int seg = ((p.C + NW - 1) / NW + 63) & ~63;
  const int a_begin = min(c1, c0 + wave * seg), a_end = min(c1, a_begin + seg);
  const bool bad = count_segment<8>(p.ids, h, E, a_begin, a_end, lane);
  if (__ballot(bad) != 0ull && lane == 0) atomicOr(p.err, 1);
  __syncthreads();
  for (int e = tid; e < E; e += NT) p.cnt[(size_t)e * p.G + g] = h[e];
  wait_wave_stores();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (unsigned)(p.G - 1);
    if (last) __hip_atomic_store(p.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every workgroup's counts are visible

  // every workgroup's counts to LDS, 8 loads per thread in flight
  const int G = p.G;
  const int EG = E * G;
  for (int i0 = tid; i0 < EG; i0 += 8 * NT) {
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = i0 + j * NT < EG ? p.cnt[i0 + j * NT] : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (i0 + j * NT < EG) M[i0 + j * NT] = v[j];
  }
  __syncthreads();
  // totals and padded sizes (a thread per expert)
  for (int e = tid; e < E; e += NT) {
    const int* row = M + e * G;
    int c = 0;
    for (int w = 0; w < G; ++w) c += row[w];
    h[e] = (c + p.bm - 1) / p.bm * p.bm;
  }
  __syncthreads();
  if (wave == 0) {
    const int per = (E + 63) / 64;
    const int lo = min(E, lane * per);
    const int hi = min(E, lo + per);
    int run = 0;
    for (int e = lo; e < hi; ++e) run += h[e];
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int excl = incl - run;
    for (int e = lo; e < hi; ++e) {
      st[e] = excl;
      excl += h[e];
    }
    if (lane == 63) st[E] = incl;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += NT) p.start[e] = st[e];
  if (tid == 0) p.num_post_padded[0] = st[E];
  if (p.pairs) write_pair_table(st, E, p.bm, p.pairs, M + EG);
  // first slot of each (expert, workgroup): exclusive scan over g, a
  // thread per expert
  for (int e = tid; e < E; e += NT) {
    const int* row = M + e * G;
    int32_t* out = p.cnt + (size_t)e * G;
    int run = st[e];
    for (int w = 0; w < G; ++w) {
      const int c = row[w];
      out[w] = run;
      run += c;
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void align_place_kernel(Align2Params p) {
  extern __shared__ int smem[];
  const int E = p.E;
  int* cw = smem;                 // [NW][E] per-wave counts, then first slots
  int* st = smem + NW * E;        // [E + 1]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NT = NW * 64;
  const int g = blockIdx.x;
  for (int i = tid; i < NW * E; i += NT) cw[i] = 0;
  for (int e = tid; e <= E; e += NT) st[e] = p.start[e];
  __syncthreads();
  const int c0 = g * p.C, c1 = min(p.A, c0 + p.C);
  const int seg = ((p.C + NW - 1) / NW + 63) & ~63;
  const int a_begin = min(c1, c0 + wave * seg), a_end = min(c1, a_begin + seg);
  int* my = cw + wave * E;
  count_segment<8>(p.ids, my, E, a_begin, a_end, lane);  // bad ids were flagged by the count launch
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int run = p.cnt[(size_t)e * p.G + g];
    for (int w = 0; w < NW; ++w) {
      const int c = cw[w * E + e];
      cw[w * E + e] = run;
      run += c;
    }
  }
  const int total = st[E];
  const int nb = total / p.bm;
  for (int b = g * NT + tid; b < p.max_blocks; b += p.G * NT)
    p.block_expert[b] = b < nb ? expert_of_row(st, E, b * p.bm) : -1;
  __syncthreads();
  place_segment<8>(p.ids, p.sorted_ids, my, E, p.nbits, a_begin, a_end, lane);
}

}  // namespace

int align_waves(int E) { return E <= 512 ? 16 : 8; }

// one workgroup: per-wave counts, first rows, and the pair table's scan
size_t align_lds_bytes(int E) { return ((size_t)align_waves(E) * E + 2 * ((size_t)E + 1)) * sizeof(int); }

// The multi-workgroup path: T*k of at least kAlignMultiMin assignments,
// chunks of at least 2048 (a multiple of 512) and at most
// min(256, kAlignMaxCounts / E) workgroups (the last one holds every
// workgroup's counts in LDS and walks them with a thread per expert).
#ifndef MOE_ALIGN_MULTI_MIN
#define MOE_ALIGN_MULTI_MIN 12288
#endif
constexpr int kAlignMultiMin = MOE_ALIGN_MULTI_MIN;
constexpr int kAlignMultiWaves = 8;
constexpr int kAlignMaxCounts = 16384;

struct AlignSplit {
  int C, G;
};
AlignSplit align_split(int64_t A, int E) {
  int64_t gmax = kAlignMaxCounts / E;
  if (gmax > 256) gmax = 256;
  if (gmax < 1) gmax = 1;
  int64_t C = (A + gmax - 1) / gmax;
  if (C < 2048) C = 2048;
  C = (C + 511) / 512 * 512;
  return AlignSplit{(int)C, (int)((A + C - 1) / C)};
}
bool align_multi(int64_t A) { return A >= kAlignMultiMin; }
size_t align_scratch_bytes(int64_t A, int E) {
  if (!align_multi(A)) return 0;
  return align_up(((size_t)align_split(A, E).G * E + (size_t)E + 1) * sizeof(int32_t), 256);
}

moe_status align_validate(const int32_t* ids, int T, int k, int E, int block_m, const void* sorted_ids,
                          const void* block_expert, const void* num_post_padded) {
  if (T < 0 || k < 1 || k > 16 || E < 1 || E > 1024) return MOE_E_INVAL;
  if (block_m < 1 || block_m > 1024) return MOE_E_INVAL;
  if ((int64_t)T * k > (1 << 24)) return MOE_E_INVAL;
  if (!sorted_ids || !block_expert || !num_post_padded) return MOE_E_INVAL;
  if (T > 0 && !ids) return MOE_E_INVAL;
  return MOE_OK;
}

AlignParams align_params(const int32_t* ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                         int32_t* block_expert, int32_t* num_post_padded, void* ws) {
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
  p.pairs = nullptr;
  p.fill_tail = true;
  return p;
}

moe_status launch_align(const int32_t* ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_post_padded, void* ws, hipStream_t stream,
                        int32_t* pairs, bool* pairs_written, bool fill_tail) {
  AlignParams p = align_params(ids, T, k, E, block_m, sorted_ids, block_expert, num_post_padded, ws);
  p.fill_tail = fill_tail;
  // the one-wave path (at most 64 assignments) leaves a pair table to its user
  if (pairs_written) *pairs_written = pairs != nullptr && p.A > 64;
  if (p.A > 64) p.pairs = pairs;
  const int nbits = p.nbits;
  if (align_multi(p.A)) {
    const AlignSplit sp = align_split(p.A, E);
    Align2Params q;
    q.ids = ids;
    q.sorted_ids = sorted_ids;
    q.block_expert = block_expert;
    q.num_post_padded = num_post_padded;
    q.err = p.err;
    q.counter = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + kAlignCounterOffset);
    q.cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + kCtrlBytes);
    q.start = q.cnt + (size_t)sp.G * E;
    q.pairs = p.pairs;
    q.A = p.A; q.E = E; q.bm = block_m; q.nbits = nbits; q.C = sp.C; q.G = sp.G;
    q.max_padded = p.max_padded; q.max_blocks = p.max_blocks;
    constexpr int NW = kAlignMultiWaves;
    align_count_kernel<NW><<<sp.G, NW * 64, ((size_t)E * sp.G + 3 * (size_t)E + 2) * sizeof(int), stream>>>(q);
    MOE_CHECK_LAUNCH();
    align_place_kernel<NW><<<sp.G, NW * 64, ((size_t)NW * E + (size_t)E + 1) * sizeof(int), stream>>>(q);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
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
size_t align_workspace_size(int T, int k, int E) { return kCtrlBytes + align_scratch_bytes((int64_t)T * k, E); }

}  // namespace moe

extern "C" moe_status moe_align(const int32_t* topk_ids, int T, int k, int E, int block_m,
                                int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_padded,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace moe;
  moe_status st = align_validate(topk_ids, T, k, E, block_m, sorted_ids, block_expert, num_post_padded);
  if (st != MOE_OK) return st;
  if (!workspace) return MOE_E_INVAL;
  if (workspace_bytes < align_workspace_size(T, k, E)) return MOE_E_WORKSPACE;
  return launch_align(topk_ids, T, k, E, block_m, sorted_ids, block_expert, num_post_padded, workspace,
                      stream);
}

extern "C" size_t moe_align_workspace_size(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return moe::align_workspace_size(T, k, E);
}
extern "C" int64_t moe_align_max_padded(int T, int k, int E, int block_m) {
  return moe::align_max_padded(T, k, E, block_m);
}
extern "C" int64_t moe_align_max_blocks(int T, int k, int E, int block_m) {
  return moe::align_max_blocks(T, k, E, block_m);
}
