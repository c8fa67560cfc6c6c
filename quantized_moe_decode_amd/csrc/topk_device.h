// Top-k routing by one wave per token (gfx950, wave64): a sorting network
// per lane, then k rounds of a DPP wave maximum over the lanes' heads, and
// the renormalised softmax weights.  Shared by the routing kernels of the
// single-token and the batched decode paths.
//
// Reading (hipfire expert-offload explainer, section "125GB 的 MoE 模型，
// 为什么 32GB 显卡也有得跑？": each token activates the top 8 of a layer's
// routed experts): selection by logit with ties to the lower expert index,
// weights = softmax over all logits renormalised over the selected k, which
// is the k-term softmax of the selected logits.
#pragma once
#include "hfq4_device.h"
#include "launch.h"

namespace hq {

// Order-preserving 32-bit key of a logit: a larger float gives a larger key,
// -0 and +0 give the same key, NaN sorts below -inf (key 1), and key 0 is
// reserved for "no expert" (padding lanes).
__device__ __forceinline__ uint32_t okey(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u = (u << 1) == 0u ? 0u : u;                    // -0 -> +0
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return __builtin_isnan(f) ? 1u : k;             // selects, no branches
}
__device__ __forceinline__ float okey_value(uint32_t k) {
  return as_f32((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
template <int CTL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x124>(v));
  v = max(v, dpp_u<0x128>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Keys of one token's E logits, PER per lane (expert e = lane*PER + i),
// read 4 at a time through a bounded descriptor.  The bound is E rounded up
// to 4 (every 16-byte load lies wholly inside or wholly outside it, and the
// logit areas of the workspace leave that much room); experts past E are
// masked, lanes past the bound read zeros.  Returns whether a NaN logit was
// seen by this lane.
template <int PER>
__device__ __forceinline__ int load_keys(const float* __restrict__ logits, int E, uint32_t* key) {
  const int lane = threadIdx.x & 63;
  int nan_seen = 0;
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(logits, (uint32_t)((E + 3) & ~3) * 4u);
  u32x4 raw4[PER / 4];
#pragma unroll
  for (int i = 0; i < PER; i += 4) raw4[i / 4] = bload16(rl, (uint32_t)(lane * PER + i) * 4u);
  __builtin_amdgcn_sched_barrier(0);   // every load in flight before the first use
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const int e0 = lane * PER + i;
    const u32x4 raw = raw4[i / 4];
    const uint32_t rv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float f = as_f32(rv[t]);
      const bool valid = e0 + t < E;
      key[i + t] = valid ? okey(f) : 0u;
      nan_seen |= valid & __builtin_isnan(f);
    }
  }
  return nan_seen;
}

// Sorting networks (Batcher's odd-even merge sort) for a lane's PER keys.
__device__ constexpr int SORT4[][2] = {{0, 1}, {2, 3}, {0, 2}, {1, 3}, {1, 2}};
__device__ constexpr int SORT8[][2] = {{0, 1}, {2, 3}, {4, 5}, {6, 7}, {0, 2}, {1, 3}, {4, 6},
                                       {5, 7}, {1, 2}, {5, 6}, {0, 4}, {1, 5}, {2, 6}, {3, 7},
                                       {2, 4}, {3, 5}, {1, 2}, {3, 4}, {5, 6}};
__device__ constexpr int SORT16[][2] = {
    {0, 1},  {2, 3},   {4, 5},   {6, 7},   {8, 9},   {10, 11}, {12, 13}, {14, 15}, {0, 2},
    {1, 3},  {4, 6},   {5, 7},   {8, 10},  {9, 11},  {12, 14}, {13, 15}, {1, 2},   {5, 6},
    {9, 10}, {13, 14}, {0, 4},   {1, 5},   {2, 6},   {3, 7},   {8, 12},  {9, 13},  {10, 14},
    {11, 15}, {2, 4},  {3, 5},   {10, 12}, {11, 13}, {1, 2},   {3, 4},   {5, 6},   {9, 10},
    {11, 12}, {13, 14}, {0, 8},  {1, 9},   {2, 10},  {3, 11},  {4, 12},  {5, 13},  {6, 14},
    {7, 15}, {4, 8},   {5, 9},   {6, 10},  {7, 11},  {2, 4},   {3, 5},   {6, 8},   {7, 9},
    {10, 12}, {11, 13}, {1, 2},  {3, 4},   {5, 6},   {7, 8},   {9, 10},  {11, 12}, {13, 14}};

// One comparator on composite entries (key << 32 | PER-1-i): the larger
// composite is "before" -- the larger key, or the lower expert on equal
// keys -- so one 64-bit compare orders (key, expert) pairs.
template <int PER>
__device__ __forceinline__ void local_sort(uint64_t* c) {
  constexpr int N = PER == 4 ? 5 : PER == 8 ? 19 : 63;
#pragma unroll
  for (int t = 0; t < N; ++t) {
    const int a = PER == 4 ? SORT4[t][0] : PER == 8 ? SORT8[t][0] : SORT16[t][0];
    const int b = PER == 4 ? SORT4[t][1] : PER == 8 ? SORT8[t][1] : SORT16[t][1];
    const bool sw = c[b] > c[a];
    const uint64_t ca = c[a];
    c[a] = sw ? c[b] : ca;
    c[b] = sw ? ca : c[b];
  }
}

// Four bits per sorted entry: the entry's position in the lane's block of
// experts (a 32-bit word up to 8 entries, 64-bit for 16).
template <int PER>
struct PosPack {
  typedef uint32_t T;
};
template <>
struct PosPack<16> {
  typedef uint64_t T;
};

// Top-k of one token's E logits by one wave, exactly in f32 order with ties
// to the lower expert index (PER >= ceil(E/64) logits per lane, expert e =
// lane*PER + i).
//  1. every lane sorts its PER (key, expert) entries by (key desc, expert
//     asc) with a sorting network;
//  2. k rounds: the wave maximum of the lanes' heads (DPP), the lowest lane
//     holding it wins (lower lanes hold lower experts), lane j records the
//     round-j winner and the winning lane drops its head;
//  3. weights exp(l_j - l_0) / sum_m exp(l_m - l_0), the sum taken by DPP in a
//     fixed order.
// k rounds of one reduction each replace a bit-serial threshold search:
// the dependent chain per token is k wave reductions long.
// Lanes j < k end with the j-th expert and its weight.  k <= 16.  A caller
// that needs only the first `rounds` < k experts stops there: lanes
// j < rounds get them (the same as the full run's), and no weights.
template <int PER>
__device__ void topk_keys(const uint32_t* key, int E, int k, int rounds, int& sel_e, float& sel_w,
                          uint64_t* trace) {
  const int lane = threadIdx.x & 63;
  uint64_t c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) c[i] = ((uint64_t)key[i] << 32) | (uint32_t)(PER - 1 - i);
  local_sort<PER>(c);
  // keys in order, positions packed (the winner's expert is lane*PER + pos)
  typedef typename PosPack<PER>::T P;
  uint32_t kk[PER];
  P pos = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    kk[i] = (uint32_t)(c[i] >> 32);
    pos |= (P)(PER - 1 - (uint32_t)c[i]) << (4 * i);
  }
  trace_point(trace, TK_TOPK, 2);
  uint32_t mk = 0, me = 0xFFFFFFFFu;     // lanes >= k hold "after everything"
  for (int j = 0; j < rounds; ++j) {
    const uint32_t m = wave_max_u32(kk[0]);
    const uint64_t who = __ballot(kk[0] == m);
    const int wl = (int)__builtin_ctzll(who);
    const uint32_t we =
        (uint32_t)(wl * PER) + ((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pos, wl) & 15u);
    if (lane == j) {
      mk = m;
      me = we;
    }
    const bool pop = lane == wl;
#pragma unroll
    for (int i = 0; i < PER - 1; ++i) kk[i] = pop ? kk[i + 1] : kk[i];
    kk[PER - 1] = pop ? 0u : kk[PER - 1];   // key 0: no expert
    pos = pop ? pos >> 4 : pos;
  }
  trace_point(trace, TK_TOPK, 4);
  sel_e = lane < rounds ? (int)me : -1;
  sel_w = 0.f;
  if (rounds < k) return;
  // 3. weights
  const float l = okey_value(mk);
  const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), 0));
  float ex = 0.f;
  if (lane < k) ex = (l0 == -INFINITY) ? 1.f : expf(l - l0);
  float sum = ex + dpp<0xB1>(ex);
  sum += dpp<0x4E>(sum);
  sum += dpp<0x141>(sum);
  if (k > 8) sum += dpp<0x128>(sum);   // lanes 0-7 add lanes 8-15
  sum = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 0));
  sel_w = ex / sum;
  trace_point(trace, TK_TOPK, 1);
}

// Top-k of one token's E logits (global memory) by one wave (the first
// `rounds` of them, see topk_keys).  Returns whether a NaN logit was seen.
template <int PER>
__device__ bool topk_wave(const float* __restrict__ logits, int E, int k, int rounds, int& sel_e,
                          float& sel_w, uint64_t* trace) {
  uint32_t key[PER];
  const int nan_seen = load_keys<PER>(logits, E, key);
  trace_point(trace, TK_TOPK, 0);
  topk_keys<PER>(key, E, k, rounds, sel_e, sel_w, trace);
  return __any(nan_seen);
}

__device__ bool topk_any(const float* logits, int E, int k, int rounds, int& e, float& w,
                         uint64_t* trace) {
  if (E <= 256) return topk_wave<4>(logits, E, k, rounds, e, w, trace);
  if (E <= 512) return topk_wave<8>(logits, E, k, rounds, e, w, trace);
  return topk_wave<16>(logits, E, k, rounds, e, w, trace);
}

}  // namespace hq
