// Top-k routing by one wave per token (gfx950, wave64): radix select of
// the k-th largest logit key, compaction, DPP bitonic sort, renormalised
// softmax weights.  Shared by the routing kernels of the single-token and
// the batched decode paths.
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
  if (__builtin_isnan(f)) return 1u;
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u << 1) == 0u) u = 0u;                     // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<0xB1>(v));
  v = min(v, dpp_u<0x4E>(v));
  v = min(v, dpp_u<0x124>(v));
  v = min(v, dpp_u<0x128>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return min(min(r0, r1), min(r2, r3));
}

// (key, index) order of the top-k: larger key first, equal keys -> lower index.
__device__ __forceinline__ bool before(uint32_t ak, uint32_t ae, uint32_t bk, uint32_t be) {
  return (ak > bk) | ((ak == bk) & (ae < be));
}
template <int CTL>
__device__ __forceinline__ void bitonic_step(uint32_t& key, uint32_t& e, bool keep_first) {
  const uint32_t pk = dpp_u<CTL>(key), pe = dpp_u<CTL>(e);
  const bool mine_first = before(key, e, pk, pe);
  const bool take = keep_first != mine_first;   // keep the partner's entry
  key = take ? pk : key;
  e = take ? pe : e;
}

// Keys of one token's E logits, PER per lane (expert e = lane*PER + i),
// read through a bounded descriptor (lanes past the end read zeros).
// Returns whether a NaN logit was seen by this lane.
template <int PER>
__device__ __forceinline__ int load_keys(const float* __restrict__ logits, int E, uint32_t* key) {
  const int lane = threadIdx.x & 63;
  int nan_seen = 0;
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(logits, (uint32_t)E * 4u);
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const int e0 = lane * PER + i;
    const u32x4 raw = bload16(rl, (uint32_t)e0 * 4u);
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

// Sum over the wave of a per-lane count (uniform result, fixed order).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u<0xB1>(v);
  v += dpp_u<0x4E>(v);
  v += dpp_u<0x124>(v);
  v += dpp_u<0x128>(v);
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return (r0 + r1) + (r2 + r3);
}

// Top-k of one token's E logits by one wave, exactly in f32 order with ties
// to the lower expert index (PER >= ceil(E/64) logits per lane, expert e =
// lane*PER + i).
//  1. radix select of T, the k-th largest key, two bits per step: three
//     candidate thresholds are counted at once (per-lane counts, DPP sums);
//     the search stops as soon as exactly k keys are >= a candidate (exact ties
//     at the boundary run all 32 bits);
//  2. the winners are every key > T plus the lowest-index keys == T, up to
//     k; they are compacted (in index order) into lanes 0..k-1 through a
//     64-entry LDS table (`scratch`, 256 bytes per wave);
//  3. a bitonic network on DPP (mirror/xor partners inside 8 or 16 lanes)
//     sorts them by (key desc, index asc);
//  4. weights exp(l_j - l_0) / sum_m exp(l_m - l_0), the sum taken by DPP in a
//     fixed order.
// Lanes j < k end with the j-th expert and its weight.  k <= 16.
template <int PER>
__device__ void topk_keys(const uint32_t* key, int E, int k, int& sel_e, float& sel_w,
                          uint32_t* scratch, uint64_t* trace) {
  const int lane = threadIdx.x & 63;
  // 1. threshold
  uint32_t T = 0;
  for (int b = 30; b >= 0; b -= 2) {
    const uint32_t c1 = T | (1u << b), c2 = T | (2u << b), c3 = T | (3u << b);
    // counts per lane on the VALU (n1 | n2 << 16, and n3), then two DPP sums:
    // ballot + popcount per key would queue on the scalar unit the CU's
    // waves share
    uint32_t p12 = 0, p3 = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      p12 += (key[i] >= c1 ? 1u : 0u) + (key[i] >= c2 ? 0x10000u : 0u);
      p3 += key[i] >= c3 ? 1u : 0u;
    }
    p12 = wave_sum_u32(p12);
    const int n1 = (int)(p12 & 0xFFFFu), n2 = (int)(p12 >> 16), n3 = (int)wave_sum_u32(p3);
    T = (n3 >= k) ? c3 : (n2 >= k) ? c2 : (n1 >= k) ? c1 : T;
    if (n1 == k || n2 == k || n3 == k) break;   // exactly k keys >= T: done
  }
  trace_point(trace, TK_TOPK, 2);
  // 2. winners: keys > T, then keys == T in index order up to k
  int n_gt = 0, below_eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    n_gt += __builtin_popcountll(__ballot(key[i] > T));
    const uint64_t eq = __ballot(key[i] == T);
    below_eq += __builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
  }
  const int need = k - n_gt;
  int own_eq = 0, below_sel = 0, own_sel = 0;
  bool sel[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool is_eq = key[i] == T;
    sel[i] = key[i] > T || (is_eq && below_eq + own_eq < need);
    own_eq += is_eq;
    const uint64_t sm = __ballot(sel[i]);
    below_sel += __builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (sel[i]) {
      const int slot = below_sel + own_sel;
      scratch[slot] = key[i];
      scratch[32 + slot] = (uint32_t)(lane * PER + i);
    }
    own_sel += sel[i];
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the table is written
  __builtin_amdgcn_wave_barrier();
  uint32_t mk = 0, me = 0xFFFFFFFFu;     // lanes >= k hold "after everything"
  if (lane < k) {
    mk = scratch[lane];
    me = scratch[32 + lane];
  }
  trace_point(trace, TK_TOPK, 3);
  // 3. bitonic sort (descending) of lanes 0..15, flip variant: the first
  //    step of each merge compares mirrored partners, later steps xor
  //    partners; the lower lane of each pair keeps the entry that comes first
  const bool lo1 = (lane & 1) == 0, lo2 = (lane & 2) == 0, lo4 = (lane & 4) == 0,
             lo8 = (lane & 8) == 0;
  bitonic_step<0xB1>(mk, me, lo1);    // size 2: xor 1
  bitonic_step<0x1B>(mk, me, lo2);    // size 4: mirror in 4
  bitonic_step<0xB1>(mk, me, lo1);
  bitonic_step<0x141>(mk, me, lo4);   // size 8: mirror in 8
  bitonic_step<0x4E>(mk, me, lo2);
  bitonic_step<0xB1>(mk, me, lo1);
  if (k > 8) {
    bitonic_step<0x140>(mk, me, lo8); // size 16: mirror in 16
    // xor 4 inside 16 lanes: rotate by 4 for the upper, by 12 for the lower half of each 8
    {
      const uint32_t ak = dpp_u<0x12C>(mk), ae = dpp_u<0x12C>(me);   // lane i <- i+4 (mod 16)
      const uint32_t bk = dpp_u<0x124>(mk), be = dpp_u<0x124>(me);   // lane i <- i-4 (mod 16)
      const uint32_t pk = lo4 ? ak : bk, pe = lo4 ? ae : be;
      const bool take = lo4 != before(mk, me, pk, pe);
      mk = take ? pk : mk;
      me = take ? pe : me;
    }
    bitonic_step<0x4E>(mk, me, lo2);
    bitonic_step<0xB1>(mk, me, lo1);
  }
  trace_point(trace, TK_TOPK, 4);
  // 4. weights
  const float l = okey_value(mk);
  const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), 0));
  float ex = 0.f;
  if (lane < k) ex = (l0 == -INFINITY) ? 1.f : expf(l - l0);
  float sum = ex + dpp<0xB1>(ex);
  sum += dpp<0x4E>(sum);
  sum += dpp<0x141>(sum);
  if (k > 8) sum += dpp<0x128>(sum);   // lanes 0-7 add lanes 8-15
  sum = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sum), 0));
  sel_e = lane < k ? (int)me : -1;
  sel_w = ex / sum;
  trace_point(trace, TK_TOPK, 1);
}

// Top-k of one token's E logits (global memory) by one wave.  Returns
// whether a NaN logit was seen.
template <int PER>
__device__ bool topk_wave(const float* __restrict__ logits, int E, int k, int& sel_e, float& sel_w,
                          uint32_t* scratch, uint64_t* trace) {
  uint32_t key[PER];
  const int nan_seen = load_keys<PER>(logits, E, key);
  trace_point(trace, TK_TOPK, 0);
  topk_keys<PER>(key, E, k, sel_e, sel_w, scratch, trace);
  return __any(nan_seen);
}

__device__ bool topk_any(const float* logits, int E, int k, int& e, float& w, uint32_t* scratch,
                         uint64_t* trace) {
  if (E <= 256) return topk_wave<4>(logits, E, k, e, w, scratch, trace);
  if (E <= 512) return topk_wave<8>(logits, E, k, e, w, scratch, trace);
  return topk_wave<16>(logits, E, k, e, w, scratch, trace);
}

}  // namespace hq
