// Router: gate logits + scoring + (group limit) + top-k + renormalisation
// (one launch at decode, two at prefill).
//
// [Router] §1.1 (three steps), §1.3 (rank key = score + bias, weight = score),
// §2 (fp32 logits and bias), §5.3 (one row per wave, k rounds, lowest id wins
// ties), §8.1 (the GEMV wants expert-parallel blocks, the top-k wants
// row-parallel waves) and §9 (a token's logits must not depend on its batch).
//
// Logit arithmetic (identical for every T and both layouts below, so a
// token's logits and choice are bit-identical whatever batch it is in):
//  * the fp32 gate value g is split exactly into three bf16 planes,
//    g = hi + mid + lo (hi: g with its low 16 bits cleared; mid: the same for
//    the remainder; lo: the last <= 8 significant bits), and x is bf16, so
//    every product x * plane is exact in fp32 and v_mfma_f32_16x16x32_bf16
//    accumulates bf16(x) * fp32(gate) to fp32 accuracy; a bf16 gate (the
//    form the page's engines store, [Router] §1.1, §2.4 and §5.1: bf16
//    hidden states times bf16 gate rows into fp32 logits; half the gate
//    bytes) is its own hi plane and takes one MFMA per K step instead of
//    three (its mid and lo planes are zero);
//  * K is cut into chunks of 128; P_c = MFMA chain over chunk c from zero
//    (4 K-steps, each hi, mid, lo in that order);
//  * G_j = P_4j + P_4j+1 + P_4j+2 + P_4j+3 (left to right), and
//    logit = G_0 + G_1 + ... (left to right).
//
// Layouts:
//  * small T (decode): a workgroup owns 16 experts x one group (4 chunks, one
//    per wave) x one 16-token tile, splits its gate values in registers, sums
//    its 4 chunk partials into G_j and stores them.  One agent-scope
//    acquire-release counter per token tile elects the workgroup that arrives
//    last (nobody waits); it adds the G_j, then runs the selection for the
//    tile's tokens, one wave per token, with the E logits in VGPRs (slot s of
//    lane l is expert s*64 + l), and resets the counter.
//    With the alignment fused in (route + align in one launch), the last
//    token tile to finish (a second agent-scope counter) then runs the
//    one-workgroup block alignment over all T*k assignments.
//  * larger T or a larger gate (use_large: where the decode layout would
//    need more than one token per selecting wave): a tiled logits kernel (128 tokens x 64 experts per workgroup,
//    each gate value split once per 128 tokens into LDS planes) writes fp32
//    logits, then a row-parallel kernel runs the same selection, one wave per
//    token.

#include "align_block.h"
#include "common.h"
#include "launch.h"
#include "quant.h"

namespace moe {

namespace {

constexpr int KCH = 128;          // K chunk
constexpr int CPG = 4;            // chunks per group
constexpr int PROW = 104;         // LDS plane row (bf16): hi[32] mid[32] lo[32] pad[8]
// The decode layout takes tiles of 4 tokens (one per wave of the selecting
// workgroup; each tile reads the whole gate) and serves T <= 4, and T <= 64
// while those tiles read at most 24 MiB of gate in all; one election
// counter per tile.  Measured (cold, router alone): where it needs more
// tokens per wave (16-token tiles) the two-launch prefill layout is faster:
// DSV3 T=256 128 -> 24 us, DSV4 T=256 74 -> 21 us, GLM T=256 83 -> 21 us,
// Qwen3 T=256 26.5 -> 19.7 us, while with 4-token tiles the decode layout
// wins (Qwen3 T=64 16.1 against 18.6, DSV3 T=8 19.4 against about 23).
constexpr int SMALL_T_TILE4 = 64;
constexpr double TILE4_GATE_BYTES = 24.0 * 1024 * 1024;
static_assert(SMALL_T_TILE4 / 4 <= kMaxCounters, "router counters");

struct RouteParams {
  const uint16_t* x;
  const void* gate;  // fp32 [E, H], or bf16 [E, H] in the GB kernels
  const float* bias;
  float* part;        // decode layout: group sums [NG][T][E]
  float* logits_out;  // optional [T][E]
  unsigned* counters;
  int32_t* ids;
  float* weights;
  int T, H, E, k, n_group, topk_group, scoring, renorm;
  int n_shared;  // 1: slot k of every token is the shared expert (id E, weight 1)
  int ks;        // ids / weights row stride, k + n_shared
  float scale;
  // decode layout in a layer call: also quantise x for the FP8 (1) or MX (2)
  // expert GEMMs into xq [T, H] e4m3 and xs (fp32 [T, H/128] or e8m0
  // [T, H/32]); 0: not
  uint8_t* xq;
  void* xs;
  int qfmt;
  int NF, NC, NG;
  int tt;  // decode layout: tokens per token tile (16 rows of the MFMA tile, the rest padding)
};

// g = hi + mid + lo exactly, each a bf16 (returned as the upper 16 bits).
__device__ __forceinline__ void split3(float g, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t h = __float_as_uint(g) & 0xFFFF0000u;
  const float r = g - __uint_as_float(h);
  const uint32_t m = __float_as_uint(r) & 0xFFFF0000u;
  const float l = r - __uint_as_float(m);
  hi = h >> 16;
  mid = m >> 16;
  lo = __float_as_uint(l) >> 16;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, v);
}

// 8 consecutive fp32 gate values -> the three bf16x8 MFMA operands
__device__ __forceinline__ void split8(const float4& g0, const float4& g1, bf16x8_t& bh, bf16x8_t& bm,
                                       bf16x8_t& bl) {
  const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split3(g[i], h[i], m[i], l[i]);
  bh = as_bf16x8(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  bm = as_bf16x8(m[0] | (m[1] << 16), m[2] | (m[3] << 16), m[4] | (m[5] << 16), m[6] | (m[7] << 16));
  bl = as_bf16x8(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}

__device__ __forceinline__ f32x4_t mfma3(const bf16x8_t& a, const bf16x8_t& bh, const bf16x8_t& bm,
                                         const bf16x8_t& bl, f32x4_t acc) {
  acc = mfma_16x16x32_bf16(a, bh, acc);
  acc = mfma_16x16x32_bf16(a, bm, acc);
  acc = mfma_16x16x32_bf16(a, bl, acc);
  return acc;
}

// The K step of one 16 x 16 logit tile: three planes of an fp32 gate, or the
// one plane of a bf16 gate (GB).
template <bool GB>
__device__ __forceinline__ f32x4_t gate_step(const bf16x8_t& a, const bf16x8_t& bh, const bf16x8_t& bm,
                                             const bf16x8_t& bl, f32x4_t acc) {
  if constexpr (GB) return mfma_16x16x32_bf16(a, bh, acc);
  return mfma3(a, bh, bm, bl, acc);
}

// Selection for one token from its E fp32 logits (l[s] = logit of expert
// s*64 + lane, -inf past E); writes ids / weights of token t.  Every
// arg-max is a wave max of the keys (DPP) followed by one ballot per slot
// for the lowest expert id holding that key.
// sid (optional, LDS): the token's k ids are also stored there.
template <int SLOTS>
__device__ __forceinline__ void select_token(const RouteParams& p, int t, const float (&l)[SLOTS],
                                             const float (&bv)[SLOTS], int* sid = nullptr) {
  const int lane = threadIdx.x & 63;
  float key[SLOTS], sc[SLOTS];
  bool ok[SLOTS];
  const float NEG_INF = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) ok[s] = s * kWave + lane < p.E;

  if (p.scoring == MOE_SOFTMAX) {
    float m = NEG_INF;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) m = fmaxf(m, l[s]);
    m = wave_max_u(m);
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      sc[s] = ok[s] ? expf(l[s] - m) : 0.f;
      part += sc[s];
    }
    const float inv = 1.f / wave_sum_u(part);
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      sc[s] = sc[s] * inv;
      key[s] = ok[s] ? sc[s] : NEG_INF;
    }
  } else if (p.scoring == MOE_SIGMOID) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      sc[s] = 1.f / (1.f + expf(-l[s]));
      key[s] = ok[s] ? sc[s] + bv[s] : NEG_INF;
    }
  } else {  // sqrt(softplus), softplus(l) = max(l, 0) + log1p(exp(-|l|))
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      sc[s] = sqrtf(fmaxf(l[s], 0.f) + log1pf(expf(-fabsf(l[s]))));
      key[s] = ok[s] ? sc[s] + bv[s] : NEG_INF;
    }
  }

  if (p.n_group > 1) {
    // group score = sum of the two largest rank keys of the group (a tie at
    // the top counts twice)
    const int gsize = p.E / p.n_group;
    int grp[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) grp[s] = ok[s] ? (s * kWave + lane) / gsize : -1;
    float my_gs = NEG_INF;
    if (gsize == 32 && p.E == SLOTS * kWave) {
      // every group is one half of one slot (DeepSeek-V3: 8 x 32): all
      // groups at once, half-wave maxima of each slot; the same maxima, the
      // same lowest-id drop and the same sums as the loop below
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const float r1 = row_max16(key[s]);
        const float lo1 = fmaxf(readlane_f32(r1, 0), readlane_f32(r1, 16));
        const float hi1 = fmaxf(readlane_f32(r1, 32), readlane_f32(r1, 48));
        const uint64_t b = __ballot(key[s] == (lane < 32 ? lo1 : hi1));
        const int dlo = __ffsll((unsigned long long)(b & 0xFFFFFFFFull)) - 1;
        const int dhi = __ffsll((unsigned long long)(b >> 32)) + 31;
        const float r2 = row_max16(lane == (lane < 32 ? dlo : dhi) ? NEG_INF : key[s]);
        const float lo2 = fmaxf(readlane_f32(r2, 0), readlane_f32(r2, 16));
        const float hi2 = fmaxf(readlane_f32(r2, 32), readlane_f32(r2, 48));
        if (lane == 2 * s) my_gs = lo1 + lo2;
        if (lane == 2 * s + 1) my_gs = hi1 + hi2;
      }
    } else {
      for (int g = 0; g < p.n_group; ++g) {
        float v = NEG_INF;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
          if (grp[s] == g) v = fmaxf(v, key[s]);
        const float t1 = wave_max_u(v);
        int drop = -1;  // lowest expert of the group holding t1
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
          const uint64_t b = __ballot(grp[s] == g && key[s] == t1);
          if (drop < 0 && b != 0) drop = s * kWave + __ffsll((unsigned long long)b) - 1;
        }
        float v2 = NEG_INF;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
          if (grp[s] == g && s * kWave + lane != drop) v2 = fmaxf(v2, key[s]);
        const float t2 = wave_max_u(v2);
        if (lane == g) my_gs = t1 + t2;
      }
    }
    // keep the topk_group best groups, lowest group id on ties
    uint64_t kept = 0;
    bool g_used = lane >= p.n_group;
    for (int r = 0; r < p.topk_group; ++r) {
      const float m = wave_max_u(g_used ? NEG_INF : my_gs);
      const uint64_t b = __ballot(!g_used && my_gs == m);
      const int g = b != 0 ? __ffsll((unsigned long long)b) - 1 : 0;
      kept |= 1ull << g;
      if (lane == g) g_used = true;
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s)
      if (ok[s] && !((kept >> grp[s]) & 1ull)) ok[s] = false;
  }

  // k rounds of arg-max on (key descending, id ascending); an expert that is
  // not allowed or already taken has key -inf (every allowed key is finite)
#pragma unroll
  for (int s = 0; s < SLOTS; ++s)
    if (!ok[s]) key[s] = NEG_INF;
  int sel_id = 0;
  float sel_s = 0.f;
  for (int j = 0; j < p.k; ++j) {
    float v = key[0];
#pragma unroll
    for (int s = 1; s < SLOTS; ++s) v = fmaxf(v, key[s]);
    const float m = wave_max_u(v);
    int id = 0;
#pragma unroll
    for (int s = SLOTS - 1; s >= 0; --s) {  // the lowest slot with a hit wins
      const uint64_t b = __ballot(key[s] == m);
      if (b != 0) id = s * kWave + __ffsll((unsigned long long)b) - 1;
    }
    const int sl = id >> 6, ln = id & 63;
    float sv = sc[0];
#pragma unroll
    for (int s = 1; s < SLOTS; ++s)
      if (s == sl) sv = sc[s];
    const float s_w = readlane_f32(sv, ln);
    if (lane == ln) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
        if (s == sl) key[s] = NEG_INF;
    }
    if (lane == j) { sel_id = id; sel_s = s_w; }
  }
  float wgt = sel_s;
  if (p.renorm) {
    const float sum = wave_sum_u(lane < p.k ? sel_s : 0.f);
    wgt = sel_s / (sum + 1e-20f);
  }
  wgt *= p.scale;
  if (p.n_shared && lane == p.k) {  // the shared expert: an always-selected slot
    sel_id = p.E;
    wgt = 1.f;
  }
  if (lane < p.ks) {
    p.ids[(size_t)t * p.ks + lane] = sel_id;
    p.weights[(size_t)t * p.ks + lane] = wgt;
    if (sid) sid[lane] = sel_id;
  }
}

// Selection bias of the lane's experts (0 without a bias or past E).
template <int SLOTS>
__device__ __forceinline__ void load_bias(const RouteParams& p, float (&bv)[SLOTS]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int e = s * kWave + lane;
    bv[s] = (p.bias != nullptr && e < p.E) ? p.bias[e] : 0.f;
  }
}

// logit of token t = G_0 + G_1 + ... (left to right) from the group sums
// part[j][t][e]; -inf past E; also stored to logits_out if requested.  The
// group sums are loaded 8 groups at a time (all in flight together).
template <int SLOTS>
__device__ __forceinline__ void sum_groups(const RouteParams& p, int t, float (&l)[SLOTS]) {
  const int lane = threadIdx.x & 63;
  int ec[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    ec[s] = min(s * kWave + lane, p.E - 1);
    l[s] = p.part[(size_t)t * p.E + ec[s]];
  }
  // U groups' sums in flight at once (64 VGPRs of them)
  constexpr int U = SLOTS <= 4 ? 16 : (64 / SLOTS < 4 ? 4 : 64 / SLOTS);
  for (int j0 = 1; j0 < p.NG; j0 += U) {
    float pv[U][SLOTS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = min(j0 + u, p.NG - 1);
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) pv[u][s] = p.part[((size_t)jj * p.T + t) * p.E + ec[s]];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u < p.NG) {
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) l[s] += pv[u][s];
      }
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int e = s * kWave + lane;
    if (e >= p.E) l[s] = -__builtin_inff();
    else if (p.logits_out) p.logits_out[(size_t)t * p.E + e] = l[s];
  }
}

// Activation quantisation of one 128-wide K chunk of token t, from the x
// fragments a wave holds for its MFMA steps (lane (r, q) holds x[t, c*128 +
// 32 s + 8 q .. +8] for s < 4): for FP8 the chunk is one group, for MX each
// s is one group of 32.  Same arithmetic as the quantisation kernel.
__device__ __forceinline__ void quant_chunk(const RouteParams& p, int t, bool tv, int c, int q,
                                            const bf16x8_t (&a)[4]) {
  float v[4][8];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4_t u = __builtin_bit_cast(u32x4_t, a[s]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[s][2 * i] = bf16_lo(u[i]);
      v[s][2 * i + 1] = bf16_hi(u[i]);
    }
  }
  uint8_t* xq = p.xq + (size_t)t * p.H + c * KCH + 8 * q;
  // FP8 divides by the group's scale, MX multiplies by its exact inverse
  // (the arithmetic of quant_x_kernel)
  auto store8 = [&](int s, float sc, bool divide) {
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = divide ? fp8_scaled(v[s][i], sc) : clamp448(v[s][i] * sc);
    uint2 w;
    w.x = pack4_e4m3(g[0], g[1], g[2], g[3]);
    w.y = pack4_e4m3(g[4], g[5], g[6], g[7]);
    *reinterpret_cast<uint2*>(xq + 32 * s) = w;
  };
  if (p.qfmt == 1) {
    float m = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[s][i]));
    m = fmaxf(m, __shfl_xor(m, 16, kWave));  // the 4 lanes of a token row
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    const float sc = fp8_group_scale(m);
    if (tv) {
#pragma unroll
      for (int s = 0; s < 4; ++s) store8(s, sc, true);
      if (q == 0) static_cast<float*>(p.xs)[(size_t)t * (p.H / KCH) + c] = sc;
    }
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[s][i]));
      m = fmaxf(m, __shfl_xor(m, 16, kWave));
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      const uint32_t code = mx_group_code(m);
      if (tv) {
        store8(s, e8m0_inv(code), false);
        if (q == 0) static_cast<uint8_t*>(p.xs)[(size_t)t * (p.H / 32) + c * 4 + s] = (uint8_t)code;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode layout.  grid.x = NF * NG (expert fragment, group), grid.y = token
// tiles of p.tt = 4 tokens, so that each wave of the elected workgroup
// selects one token (the selection is single-wave VALU code; measured:
// 4-token against 16-token tiles took the Qwen3 router at T=16 from 16.0 to
// 8.7 us and DSV3's at T=8 from 23.2 to 18.7 us).  FUSE (one token tile
// only): the selecting workgroup also aligns, from the ids it keeps in LDS
// (one wave for at most 64 assignments, else dynamic LDS of (5 E + 1) ints,
// E counting the shared expert).
template <int SLOTS, bool FUSE, bool GB>
__global__ __launch_bounds__(256) void route_small(RouteParams p, AlignParams ap) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int f = blockIdx.x % p.NF;
  const int j = blockIdx.x / p.NF;
  const int ttile = blockIdx.y;
  const int t0 = ttile * p.tt;
  const int c = j * CPG + wave;
  __shared__ float red[CPG][16][17];
  __shared__ int s_last;
  __shared__ int s_ids[FUSE ? 16 * 17 : 1];  // FUSE: the tile's ids [tokens][k + n_shared]

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (c < p.NC) {
    const int e = min(f * 16 + r, p.E - 1);
    const size_t goff = (size_t)e * p.H + c * KCH + q * 8;
    const int t = t0 + r;
    const bool tv = r < p.tt && t < p.T;
    const uint16_t* xrow = p.x + (size_t)(tv ? t : 0) * p.H + c * KCH + q * 8;
    float4 g0[4], g1[4];
    bf16x8_t gb[4];
    bf16x8_t a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (GB) {
        gb[s] = *reinterpret_cast<const bf16x8_t*>(static_cast<const uint16_t*>(p.gate) + goff + 32 * s);
      } else {
        const float* grow = static_cast<const float*>(p.gate) + goff;
        g0[s] = *reinterpret_cast<const float4*>(grow + 32 * s);
        g1[s] = *reinterpret_cast<const float4*>(grow + 32 * s + 4);
      }
      a[s] = *reinterpret_cast<const bf16x8_t*>(xrow + 32 * s);
      if (!tv) a[s] = bf16x8_t{};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t bh, bm, bl;
      if constexpr (GB) bh = gb[s];
      else split8(g0[s], g1[s], bh, bm, bl);
      acc = gate_step<GB>(a[s], bh, bm, bl, acc);
    }
    // the workgroups of expert fragment 0 cover every chunk of the tile once
    if (p.qfmt != 0 && f == 0) quant_chunk(p, t, tv, c, q, a);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * q + i][r] = acc[i];
  __syncthreads();
  if (wave == 0) {
    const int nc = min(CPG, p.NC - j * CPG);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = lane * 4 + i;  // 256 entries of the 16 x 16 tile
      const int tl = idx >> 4;
      const int el = idx & 15;
      float gsum = red[0][tl][el];
      for (int w = 1; w < nc; ++w) gsum += red[w][tl][el];
      const int t = t0 + tl;
      const int e = f * 16 + el;
      // written through to memory (system scope): the election's release
      // then has fewer dirty L2 lines to write back (measured: the router
      // alone 0.3-1 us faster)
      if (tl < p.tt && t < p.T && e < p.E)
        __hip_atomic_store(p.part + ((size_t)j * p.T + t) * p.E + e, gsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
  __syncthreads();  // only wave 0 (thread 0's wave) stored group sums
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(p.counters + ttile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (unsigned)(gridDim.x - 1);
    if (last) __hip_atomic_store(p.counters + ttile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every wave sees all group sums
  for (int tl = wave; tl < p.tt; tl += 4) {
    const int t = t0 + tl;
    if (t >= p.T) break;
    float bv[SLOTS];
    load_bias<SLOTS>(p, bv);
    float l[SLOTS];
    sum_groups<SLOTS>(p, t, l);
    select_token<SLOTS>(p, t, l, bv, FUSE ? s_ids + tl * p.ks : nullptr);
  }
  if constexpr (FUSE) {
    extern __shared__ int smem[];
    // one token tile (the host fuses only then): this workgroup selected
    // every token and aligns from the ids it keeps in LDS
    __syncthreads();
    AlignParams lp = ap;
    lp.ids = s_ids;
    if (lp.A <= 64)
      align_tiny<4>(lp);
    else
      align_block<4>(lp, smem);
  }
}

// ---------------------------------------------------------------------------
// Prefill layout, first kernel: the group sum G_j of a 128-token x 32 EW-expert
// tile for one K group j (4 chunks of 128), written to part[j][t][e].
// 4 waves as 2 x 2, each 64 tokens x 16 EW experts (4 x EW fragments).  Per
// 32-wide K step the 256 threads split the tile's 32 EW x 32 gate values once
// into LDS planes (each gate value is split once per 128 tokens: the split
// and its two barriers per step cost more than the step's multiplies at
// 64 tokens); the gate and x values of the next PF steps are in flight
// meanwhile.
constexpr int TFR = 4;             // token fragments per wave
constexpr int LT = 2 * 16 * TFR;   // tokens per tile
constexpr int PF = 1;   // steps loaded ahead (measured: 1 against 4, the same
                        // at Qwen3 T=4096 and GLM T=512, DSV3 T=2048 66.9 -> 60.5 us,
                        // DSV4 T=8192 115.5 -> 101.1 us: fewer registers, more
                        // workgroups per CU)
// Expert fragments per wave: a tile holds 32 EW experts, and each expert
// tile reads the token rows' x once.  EW = 4 (227 VGPRs, two waves per SIMD)
// where its grid still has at least kWideTiles workgroups, else 2 (142
// VGPRs, three).  Measured (router alone, warm, EW 2 against 4): DSV4 T=8192
// 114.5 / 98 us (1024 wide tiles), DSV3 T=2048 64.7 / 56 us (448), but Qwen3
// T=4096 35 / 43.5 (128), GLM T=512 32 / 39.7 (96), DSV3 T=256 33 / 41 (56).
constexpr int kWideTiles = 384;

template <bool GB, int EW>
__global__ __launch_bounds__(256) void route_logits_group(RouteParams p) {
  constexpr int LE = 32 * EW;  // experts per tile
  __shared__ __attribute__((aligned(16))) uint16_t planes[LE * PROW];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int t0 = blockIdx.x * LT;
  const int e0 = blockIdx.y * LE;
  const int j = blockIdx.z;                     // K group
  const int k0 = j * KCH * CPG;                 // first K of the group
  const int nsteps = min(KCH * CPG, p.H - k0) / 32;

  // this thread's EW pieces of four gate values per K step: expert rows
  // (tid >> 3) + 32 i, K offset (tid & 7) * 4
  const int se = tid >> 3;
  const int sk = (tid & 7) * 4;
  bool sv[EW];
  size_t go[EW];
#pragma unroll
  for (int i = 0; i < EW; ++i) {
    sv[i] = e0 + se + 32 * i < p.E;
    go[i] = (size_t)min(e0 + se + 32 * i, p.E - 1) * p.H + k0 + sk;
  }
  const float* g32 = static_cast<const float*>(p.gate);
  const uint16_t* g16 = static_cast<const uint16_t*>(p.gate);
  const uint16_t* xr[TFR];
  bool tv[TFR];
#pragma unroll
  for (int tf = 0; tf < TFR; ++tf) {
    const int t = t0 + wm * (LT / 2) + tf * 16 + r;
    tv[tf] = t < p.T;
    xr[tf] = p.x + (size_t)(tv[tf] ? t : 0) * p.H + k0 + q * 8;
  }

  f32x4_t part[TFR][EW], grp[TFR][EW];
#pragma unroll
  for (int a = 0; a < TFR; ++a)
#pragma unroll
    for (int b = 0; b < EW; ++b) {
      part[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      grp[a][b] = part[a][b];
    }

  // register ring of PF steps (past the last step: the last step again), as
  // raw bits: four fp32 gate values per row, or four bf16 ones in .x / .y
  uint4 rg[PF][EW];
  bf16x8_t rx[PF][TFR];
  auto load = [&](int st, int slot) {
    const int kb = min(st, nsteps - 1) * 32;
#pragma unroll
    for (int i = 0; i < EW; ++i) {
      if constexpr (GB) {
        const uint2 v = *reinterpret_cast<const uint2*>(g16 + go[i] + kb);
        rg[slot][i] = make_uint4(v.x, v.y, 0u, 0u);
      } else {
        rg[slot][i] = *reinterpret_cast<const uint4*>(g32 + go[i] + kb);
      }
    }
#pragma unroll
    for (int tf = 0; tf < TFR; ++tf) rx[slot][tf] = *reinterpret_cast<const bf16x8_t*>(xr[tf] + kb);
  };
#pragma unroll
  for (int u = 0; u < PF; ++u) load(u, u);

  for (int s0 = 0; s0 < nsteps; s0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int st = s0 + u;
      if (st >= nsteps) break;
      uint4 gv[EW];
#pragma unroll
      for (int i = 0; i < EW; ++i) gv[i] = sv[i] ? rg[u][i] : make_uint4(0u, 0u, 0u, 0u);
      bf16x8_t a[TFR];
#pragma unroll
      for (int tf = 0; tf < TFR; ++tf) a[tf] = tv[tf] ? rx[u][tf] : bf16x8_t{};
      load(st + PF, u);
      __syncthreads();  // the previous step's planes are consumed
#pragma unroll
      for (int i = 0; i < EW; ++i) {
        uint16_t* row = planes + (se + 32 * i) * PROW + sk;
        if constexpr (GB) {  // the bf16 gate is the hi plane
          *reinterpret_cast<uint2*>(row) = make_uint2(gv[i].x, gv[i].y);
        } else {
          uint32_t h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
          split3(__uint_as_float(gv[i].x), h0, m0, l0);
          split3(__uint_as_float(gv[i].y), h1, m1, l1);
          split3(__uint_as_float(gv[i].z), h2, m2, l2);
          split3(__uint_as_float(gv[i].w), h3, m3, l3);
          *reinterpret_cast<uint2*>(row) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
          *reinterpret_cast<uint2*>(row + 32) = make_uint2(m0 | (m1 << 16), m2 | (m3 << 16));
          *reinterpret_cast<uint2*>(row + 64) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
        }
      }
      __syncthreads();
#pragma unroll
      for (int ef = 0; ef < EW; ++ef) {
        const uint16_t* pr = planes + (wn * 16 * EW + ef * 16 + r) * PROW + q * 8;
        const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(pr);
        bf16x8_t bm{}, bl{};
        if constexpr (!GB) {
          bm = *reinterpret_cast<const bf16x8_t*>(pr + 32);
          bl = *reinterpret_cast<const bf16x8_t*>(pr + 64);
        }
#pragma unroll
        for (int tf = 0; tf < TFR; ++tf) part[tf][ef] = gate_step<GB>(a[tf], bh, bm, bl, part[tf][ef]);
      }
      if ((st & 3) == 3 || st == nsteps - 1) {  // end of a chunk: G_j += P_c (P_c from zero)
        const bool first = st < 4;
#pragma unroll
        for (int tf = 0; tf < TFR; ++tf)
#pragma unroll
          for (int ef = 0; ef < EW; ++ef) {
            grp[tf][ef] = first ? part[tf][ef] : grp[tf][ef] + part[tf][ef];
            part[tf][ef] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
  }
#pragma unroll
  for (int tf = 0; tf < TFR; ++tf)
#pragma unroll
    for (int ef = 0; ef < EW; ++ef)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int t = t0 + wm * (LT / 2) + tf * 16 + 4 * q + ii;
        const int e = e0 + wn * 16 * EW + ef * 16 + r;
        if (t < p.T && e < p.E) p.part[((size_t)j * p.T + t) * p.E + e] = grp[tf][ef][ii];
      }
}

// Prefill layout, second kernel: one wave per token selects from its logits.
template <int SLOTS>
__global__ __launch_bounds__(256) void route_select(RouteParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  float l[SLOTS], bv[SLOTS];
  load_bias<SLOTS>(p, bv);
  sum_groups<SLOTS>(p, t, l);
  select_token<SLOTS>(p, t, l, bv);
}

bool use_large(int T, int E, int H) {
  return !(T <= 4 || (T <= SMALL_T_TILE4 && (double)ceil_div(T, 4) * E * H * sizeof(float) <= TILE4_GATE_BYTES));
}

// ap: the alignment to fuse into the decode layout, or nullptr
template <int SLOTS, bool GB>
moe_status launch_slots(const RouteParams& p, const AlignParams* ap, hipStream_t stream) {
  if (use_large(p.T, p.E, p.H)) {
    const dim3 wide(ceil_div(p.T, LT), ceil_div(p.E, 128), p.NG);
    if (p.E > 64 && (int64_t)wide.x * wide.y * wide.z >= kWideTiles)
      route_logits_group<GB, 4><<<wide, 256, 0, stream>>>(p);
    else
      route_logits_group<GB, 2><<<dim3(ceil_div(p.T, LT), ceil_div(p.E, 64), p.NG), 256, 0, stream>>>(p);
    MOE_CHECK_LAUNCH();
    route_select<SLOTS><<<ceil_div(p.T, 4), 256, 0, stream>>>(p);
  } else {
    dim3 grid(p.NF * p.NG, ceil_div(p.T, p.tt));
    if (ap)  // align_block's LDS: (4 waves + 1) x the alignment's experts (E + n_shared) + 1
      route_small<SLOTS, true, GB><<<grid, 256, (5 * (size_t)ap->E + 1) * sizeof(int), stream>>>(p, *ap);
    else
      route_small<SLOTS, false, GB><<<grid, 256, 0, stream>>>(p, AlignParams{});
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace

size_t route_workspace_size(int T, int H, int E) {
  const size_t per_token = (size_t)ceil_div(H, KCH * CPG) * E;  // group sums [NG][T][E]
  return kCtrlBytes + align_up(per_token * T * sizeof(float), 256);
}

moe_status route_validate(const void* x, const void* gate, int gate_is_fp32, int T, int H, int E, int k, int n_group,
                          int topk_group, int scoring, const int32_t* ids, const float* w) {
  if (T < 0 || T > (1 << 24) || H < 128 || H % 128 != 0 || E < 1 || E > 1024 || k < 1 || k > 16 || k > E)
    return MOE_E_INVAL;
  if (scoring != MOE_SOFTMAX && scoring != MOE_SIGMOID && scoring != MOE_SQRTSOFTPLUS) return MOE_E_INVAL;
  if (gate_is_fp32 != 0 && gate_is_fp32 != 1) return MOE_E_INVAL;
  if (n_group < 1 || n_group > 64 || E % n_group != 0) return MOE_E_INVAL;
  if (n_group > 1 && (E / n_group < 2)) return MOE_E_INVAL;
  if (topk_group < 1 || topk_group > n_group) return MOE_E_INVAL;
  if ((int64_t)k > (int64_t)topk_group * (E / n_group)) return MOE_E_INVAL;
  if (T > 0 && (!x || !gate || !ids || !w)) return MOE_E_INVAL;
  return MOE_OK;
}

namespace {

template <bool GB>
moe_status launch_gate(const RouteParams& p, const AlignParams* ap, int slots, hipStream_t stream) {
  if (slots <= 1) return launch_slots<1, GB>(p, ap, stream);
  if (slots <= 2) return launch_slots<2, GB>(p, ap, stream);
  if (slots <= 4) return launch_slots<4, GB>(p, ap, stream);
  if (slots <= 5) return launch_slots<5, GB>(p, ap, stream);
  if (slots <= 8) return launch_slots<8, GB>(p, ap, stream);
  return launch_slots<16, GB>(p, ap, stream);
}

moe_status route_launch(const void* x, const void* gate, int gate_is_fp32, const float* bias, int T, int H, int E,
                        int k,
                        int n_group, int topk_group, int scoring, int renormalize, float routed_scale,
                        int n_shared, int32_t* ids, float* weights, float* logits_out, void* ws,
                        const AlignParams* ap, hipStream_t stream, void* xq = nullptr, void* xs = nullptr,
                        int qfmt = 0) {
  RouteParams p;
  p.x = static_cast<const uint16_t*>(x);
  p.gate = gate;
  p.bias = bias;
  char* base = static_cast<char*>(ws);
  p.part = reinterpret_cast<float*>(base + kCtrlBytes);
  p.logits_out = logits_out;
  p.counters = reinterpret_cast<unsigned*>(base + kCounterOffset);
  p.ids = ids;
  p.weights = weights;
  p.T = T; p.H = H; p.E = E; p.k = k;
  p.tt = 4;
  p.n_shared = n_shared; p.ks = k + n_shared;
  p.n_group = n_group; p.topk_group = topk_group;
  p.scoring = scoring; p.renorm = renormalize != 0;
  p.scale = routed_scale;
  p.xq = nullptr;
  p.xs = nullptr;
  p.qfmt = 0;
  if (qfmt != 0 && route_quantizes_x(T, E, H)) {
    p.xq = static_cast<uint8_t*>(xq);
    p.xs = xs;
    p.qfmt = qfmt;
  }
  p.NF = ceil_div(E, 16);
  p.NC = H / KCH;
  p.NG = ceil_div(p.NC, CPG);
  const int slots = ceil_div(E, kWave);
  if (gate_is_fp32) return launch_gate<false>(p, ap, slots, stream);
  return launch_gate<true>(p, ap, slots, stream);
}
}  // namespace

moe_status launch_route(const void* x, const void* gate, int gate_is_fp32, const float* bias, int T, int H, int E,
                        int k,
                        int n_group, int topk_group, int scoring, int renormalize, float routed_scale,
                        int32_t* ids, float* weights, float* logits_out, void* ws, hipStream_t stream) {
  if (T == 0) return MOE_OK;
  return route_launch(x, gate, gate_is_fp32, bias, T, H, E, k, n_group, topk_group, scoring, renormalize,
                      routed_scale, 0, ids, weights, logits_out, ws, nullptr, stream);
}

size_t route_align_workspace_size(int T, int H, int E, int k, int n_shared) {
  const size_t r = route_workspace_size(T, H, E), a = align_workspace_size(T, k + n_shared, E + n_shared);
  return r > a ? r : a;
}

// The decode layout quantises x on the way.  (The prefill layout could too,
// a 32-wide K step being one MX group, but its 32-byte pieces of each xq row
// made the layer slower: DSV4 T=8192 1868 -> 1879 us, same process.)
bool route_quantizes_x(int T, int E, int H) { return !use_large(T, E, H); }

moe_status launch_route_align(const void* x, const void* gate, int gate_is_fp32, const float* bias, int T, int H,
                              int E, int k,
                              int n_group, int topk_group, int scoring, int renormalize, float routed_scale,
                              int n_shared, int block_m, int32_t* ids, float* weights, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* num_post_padded, void* ws, hipStream_t stream,
                              void* xq, void* xs, int qfmt, int32_t* pairs, bool* pairs_written,
                              bool fill_tail) {
  // the alignment sees the shared expert as expert E and slot k
  const int Ea = E + n_shared, ka = k + n_shared;
  if (pairs_written) *pairs_written = false;
  if (T == 0) return launch_align(ids, T, ka, Ea, block_m, sorted_ids, block_expert, num_post_padded, ws, stream);
  if (!use_large(T, E, H) && T <= 4) {
    // one token tile: its selecting workgroup aligns in the same launch
    AlignParams ap = align_params(ids, T, ka, Ea, block_m, sorted_ids, block_expert, num_post_padded, ws);
    ap.fill_tail = fill_tail;
    return route_launch(x, gate, gate_is_fp32, bias, T, H, E, k, n_group, topk_group, scoring, renormalize,
                        routed_scale, n_shared, ids, weights, nullptr, ws, &ap, stream, xq, xs, qfmt);
  }
  if (!use_large(T, E, H)) {
    // several token tiles: a launch of its own aligns (measured: faster than
    // a second election among the tiles and an alignment by the last one's
    // four waves, Qwen3 T=16 route + align 15.5 against about 13 us)
    moe_status st = route_launch(x, gate, gate_is_fp32, bias, T, H, E, k, n_group, topk_group, scoring, renormalize,
                                 routed_scale, n_shared, ids, weights, nullptr, ws, nullptr, stream, xq, xs, qfmt);
    if (st != MOE_OK) return st;
    return launch_align(ids, T, ka, Ea, block_m, sorted_ids, block_expert, num_post_padded, ws, stream, pairs,
                        pairs_written, fill_tail);
  }
  moe_status st = route_launch(x, gate, gate_is_fp32, bias, T, H, E, k, n_group, topk_group, scoring, renormalize,
                               routed_scale, n_shared, ids, weights, nullptr, ws, nullptr, stream);
  if (st != MOE_OK) return st;
  return launch_align(ids, T, ka, Ea, block_m, sorted_ids, block_expert, num_post_padded, ws, stream, pairs,
                      pairs_written, fill_tail);
}

}  // namespace moe

extern "C" moe_status moe_route(const void* x, const void* gate, int gate_is_fp32, const float* bias, int T, int H,
                                int E,
                                int k, int n_group, int topk_group, int scoring, int renormalize,
                                float routed_scale, int32_t* topk_ids, float* topk_weights,
                                float* logits_out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  using namespace moe;
  moe_status st = route_validate(x, gate, gate_is_fp32, T, H, E, k, n_group, topk_group, scoring, topk_ids,
                                 topk_weights);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!workspace) return MOE_E_INVAL;
  if (workspace_bytes < route_workspace_size(T, H, E)) return MOE_E_WORKSPACE;
  return launch_route(x, gate, gate_is_fp32, bias, T, H, E, k, n_group, topk_group, scoring, renormalize, routed_scale,
                      topk_ids, topk_weights, logits_out, workspace, stream);
}

extern "C" size_t moe_route_workspace_size(int T, int H, int E) {
  if (T < 0 || H < 1 || E < 1) return 0;
  return moe::route_workspace_size(T, H, E);
}

extern "C" moe_status moe_route_align(const void* x, const void* gate, int gate_is_fp32, const float* bias, int T,
                                      int H, int E,
                                      int k, int n_shared, int n_group, int topk_group, int scoring,
                                      int renormalize, float routed_scale, int block_m, int32_t* topk_ids,
                                      float* topk_weights, int32_t* sorted_ids, int32_t* block_expert,
                                      int32_t* num_post_padded, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  using namespace moe;
  if (n_shared != 0 && n_shared != 1) return MOE_E_INVAL;
  moe_status st = route_validate(x, gate, gate_is_fp32, T, H, E, k, n_group, topk_group, scoring, topk_ids,
                                 topk_weights);
  if (st != MOE_OK) return st;
  st = align_validate(topk_ids, T, k + n_shared, E + n_shared, block_m, sorted_ids, block_expert, num_post_padded);
  if (st != MOE_OK) return st;
  if (!workspace) return MOE_E_INVAL;
  if (workspace_bytes < route_align_workspace_size(T, H, E, k, n_shared)) return MOE_E_WORKSPACE;
  return launch_route_align(x, gate, gate_is_fp32, bias, T, H, E, k, n_group, topk_group, scoring, renormalize,
                            routed_scale,
                            n_shared, block_m, topk_ids, topk_weights, sorted_ids, block_expert, num_post_padded,
                            workspace, stream, nullptr, nullptr, 0);
}

extern "C" size_t moe_route_align_workspace_size(int T, int H, int E, int k, int n_shared) {
  if (T < 0 || H < 1 || E < 1 || k < 1 || n_shared < 0 || n_shared > 1) return 0;
  return moe::route_align_workspace_size(T, H, E, k, n_shared);
}
