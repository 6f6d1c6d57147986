// Block alignment in one workgroup: the device code shared by the alignment
// kernel and the router's fused route + align launch.
//
// [MoE] "vLLM's Triton path: align, then index" and [Kernels] "Alignment:
// making ragged routing tileable": per-expert counts rounded up to whole
// blocks, exclusive scan, expert e's assignments in ascending order from its
// start, the sentinel T*k elsewhere, a block-to-expert table with -1 after
// the padded length.  Every position is decided without atomics:
//   1. each wave owns one contiguous segment of the assignments and counts its
//      ids per expert into its own LDS row cnt[w][e];
//   2. counts are summed over waves, padded to a multiple of BLOCK_M and
//      scanned (wave 0); cnt[w][e] becomes wave w's first slot for expert e;
//   3. each wave walks its segment again 64 assignments at a time; lanes with
//      equal ids find each other with one ballot per id bit, take
//      rank = #equal lanes below them, and the lowest such lane advances
//      cnt[w][e] by the group size.
#pragma once

#include "common.h"

namespace moe {

struct AlignParams {
  const int32_t* ids;
  int32_t* sorted_ids;
  int32_t* block_expert;
  int32_t* num_post_padded;
  int32_t* err;
  int A, E, bm, nbits;
  int max_padded, max_blocks;
  int32_t* pairs;  // optional: the paired GEMM tiles' pair table (write_pair_table); null: none
  // false (moe_layer, whose kernels read only below the padded length): the
  // one-wave path leaves the sentinel slots past the padded length and the
  // block table's -1 tail unwritten
  bool fill_tail;
};

// AlignParams of one call (the error word at the start of the workspace).
AlignParams align_params(const int32_t* ids, int T, int k, int E, int block_m, int32_t* sorted_ids,
                         int32_t* block_expert, int32_t* num_post_padded, void* ws);

// Pair table of the paired tiled GEMMs from the scanned first rows
// start[0..E] (LDS, start[E] = padded length): tab[0] = number of pairs,
// tab[1 + j] = pair_entry(first block of pair j, two blocks, window bits);
// an expert's blocks pair up from the first block of its run, in expert
// order (the layout pair_table_kernel writes from the block table).
// Wave 0 scans the pair counts into pb[0..E] (LDS scratch); every thread
// then writes the pairs of its experts.  Ends with a barrier.
__device__ __forceinline__ void write_pair_table(const int* start, int E, int bm, int32_t* tab, int* pb) {
  const int tid = threadIdx.x, lane = tid & 63, NT = blockDim.x;
  if (tid < 64) {
    const int per = (E + 63) / 64;
    const int lo = min(E, lane * per);
    const int hi = min(E, lo + per);
    int run = 0;
    for (int e = lo; e < hi; ++e) run += ((start[e + 1] - start[e]) / bm + 1) / 2;
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int excl = incl - run;
    for (int e = lo; e < hi; ++e) {
      pb[e] = excl;
      excl += ((start[e + 1] - start[e]) / bm + 1) / 2;
    }
    if (lane == 63) pb[E] = incl;
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    const int nb = (start[e + 1] - start[e]) / bm;
    const int b0 = start[e] / bm;
    const int m = (nb + 1) / 2;  // the expert's pairs
    for (int j = 0; j < m; ++j)
      tab[1 + pb[e] + j] = pair_entry(b0 + 2 * j, 2 * j + 1 < nb, (j & 1) == 0 && j + 1 < m, (j & 1) == 1);
  }
  if (tid == 0) tab[0] = pb[E];
  __syncthreads();
}

// expert owning padded row `row`: upper_bound of row in start[0..E], minus one
__device__ __forceinline__ int expert_of_row(const int* start, int E, int row) {
  int lo = 0, hi = E + 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (start[mid] <= row) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

// Stable placement of the assignments [a_begin, a_end) of one wave, 64 at a
// time, ids read CH per lane at once; first[e] is the wave's next slot for
// expert e (LDS, advanced here).
template <int CH>
__device__ __forceinline__ void place_segment(const int32_t* ids, int32_t* sorted_ids, int* first, int E, int nbits,
                                              int a_begin, int a_end, int lane) {
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int a1 = a_begin; a1 < a_end; a1 += 64 * CH) {
    int idv[CH];
    const int nc = min(CH, (a_end - a1 + 63) >> 6);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int a = a1 + 64 * c + lane;
      idv[c] = (c < nc && a < a_end) ? ids[a] : -1;
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {  // 64 consecutive assignments at a time, in order
      if (c >= nc) break;
      const int a = a1 + 64 * c + lane;
      int id = idv[c];
      const bool valid = id >= 0 && id < E;
      if (!valid) id = 0;
      uint64_t m = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (id >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      if (valid) {
        const int rank = __popcll(m & lt);
        const int pos = first[id] + rank;
        sorted_ids[pos] = a;
        if (rank == 0) first[id] += __popcll(m);
      }
    }
  }
}

// Count the valid ids of [a_begin, a_end) into hist (LDS atomics), CH ids
// per lane in flight; returns whether an id outside [0, E) other than -1
// was seen.
template <int CH>
__device__ __forceinline__ bool count_segment(const int32_t* ids, int* hist, int E, int a_begin, int a_end, int lane) {
  bool bad = false;
  for (int a0 = a_begin; a0 < a_end; a0 += 64 * CH) {
    int idv[CH];
    const int nc = min(CH, (a_end - a0 + 63) >> 6);  // sub-chunks of 64 holding ids
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int a = a0 + 64 * c + lane;
      idv[c] = (c < nc && a < a_end) ? ids[a] : -1;
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c >= nc) break;
      const int id = idv[c];
      if (id >= 0 && id < E)
        atomicAdd(&hist[id], 1);
      else if (id != -1)
        bad = true;
    }
  }
  return bad;
}

// Alignment of at most 64 assignments (decode) in one workgroup of NW waves.
// Wave 0 holds one assignment per lane: lanes with equal ids find each
// other with one ballot per id bit, so each lane knows its expert's count
// and its rank among them (lower assignment index first); the lowest lane
// of an expert counts the other experts' lanes with lower ids, which places
// the expert in the sorted list of distinct experts, and sums their padded
// counts, which is its first slot.  The list (first slot, count, id) goes
// to LDS; then every slot is written exactly once: an assignment by its
// lane, any other slot below the padded length by the thread that finds it
// in the list (padding of an expert) or past it (sentinel), so no store
// has to wait for another.  Same outputs as align_block.
template <int NW>
__device__ __forceinline__ void align_tiny(const AlignParams& p) {
  __shared__ int l_start[65];  // first slot of the d-th distinct expert; [D] = padded length
  __shared__ int l_count[64];
  __shared__ int l_id[64];
  __shared__ int l_d;          // D, the number of distinct experts
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int NT = NW * 64;
  const int A = p.A;
  const int E = p.E;
  if (tid < 64) {
    const int id0 = lane < A ? p.ids[lane] : -1;
    const bool valid = id0 >= 0 && id0 < E;
    if (__ballot(lane < A && !valid && id0 != -1) != 0ull && lane == 0) atomicOr(p.err, 1);
    const int id = valid ? id0 : 0;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < p.nbits; ++b) {
      const bool bit = (id >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(m & lt);
    const int cnt = __popcll(m);
    const bool lead = valid && rank == 0;
    const int padded = (cnt + p.bm - 1) / p.bm * p.bm;
    // distinct experts with lower ids than this lane's and their padded counts
    int before = 0, start = 0;
    const uint64_t leaders = __ballot(lead);
    for (uint64_t rest = leaders; rest != 0ull; rest &= rest - 1ull) {
      const int j = __ffsll((unsigned long long)rest) - 1;
      const int idj = __shfl(id, j, 64);
      const int pj = __shfl(padded, j, 64);
      if (idj < id) {
        before += 1;
        start += pj;
      }
    }
    int total = lead ? padded : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) total += __shfl_xor(total, off, 64);
    if (lead) {
      l_start[before] = start;
      l_count[before] = cnt;
      l_id[before] = id;
    }
    if (lane == 0) {
      l_d = __popcll(leaders);
      l_start[__popcll(leaders)] = total;
      p.num_post_padded[0] = total;
    }
    // every lane of an expert computed its first slot (start); plus the rank
    if (valid) p.sorted_ids[start + rank] = lane;
  }
  __syncthreads();
  const int D = l_d;
  const int total = l_start[D];
  // the distinct expert whose padded range holds slot i (i < total)
  auto owner = [&](int i) {
    int lo = 0, hi = D;  // last d with l_start[d] <= i
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (l_start[mid] <= i) lo = mid; else hi = mid;
    }
    return lo;
  };
  const int fill_end = p.fill_tail ? p.max_padded : total;
  for (int i = tid; i < fill_end; i += NT) {
    if (i < total) {
      const int d = owner(i);
      if (i - l_start[d] < l_count[d]) continue;  // an assignment's slot
    }
    p.sorted_ids[i] = A;
  }
  const int nb = total / p.bm;
  const int blk_end = p.fill_tail ? p.max_blocks : nb;
  for (int b = tid; b < blk_end; b += NT) p.block_expert[b] = b < nb ? l_id[owner(b * p.bm)] : -1;
}

// The whole alignment in one workgroup of NW waves (threadIdx.x < NW * 64);
// smem holds (NW * E + E + 1) ints, E + 1 more with a pair table.  Every slot first gets the sentinel
// (coalesced stores); the placement overwrites the assignment slots after a
// wait for those stores and a barrier.
template <int NW>
__device__ __forceinline__ void align_block(const AlignParams& p, int* smem) {
  int* cnt = smem;                   // [NW][E]
  int* start = smem + NW * p.E;      // [E + 1]
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

  for (int i = tid; i < p.max_padded; i += NT) p.sorted_ids[i] = A;
  int* my = cnt + wave * E;
  for (int e = lane; e < E; e += 64) my[e] = 0;
  // ids are read CH per lane at a time (all loads in flight together)
  constexpr int CH = 16;
  const bool bad = count_segment<CH>(p.ids, my, E, a_begin, a_end, lane);
  if (__ballot(bad) != 0ull && lane == 0) atomicOr(p.err, 1);
  __syncthreads();

  // per-expert totals and padded sizes
  for (int e = tid; e < E; e += NT) {
    int c = 0;
    for (int w = 0; w < NW; ++w) c += cnt[w * E + e];
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
  if (p.pairs) write_pair_table(start, E, p.bm, p.pairs, start + E + 1);
  // first slot of each (wave, expert)
  for (int e = tid; e < E; e += NT) {
    int run = start[e];
    for (int w = 0; w < NW; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
  }
  // block table
  const int nb = total / p.bm;
  for (int b = tid; b < p.max_blocks; b += NT) p.block_expert[b] = b < nb ? expert_of_row(start, E, b * p.bm) : -1;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the sentinel stores are done
  __syncthreads();

  // stable placement
  place_segment<CH>(p.ids, p.sorted_ids, my, E, p.nbits, a_begin, a_end, lane);
}

}  // namespace moe
