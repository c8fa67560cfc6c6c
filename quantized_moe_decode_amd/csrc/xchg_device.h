// Data exchange between the workgroups of one launch (gfx950).
//
// A word is 64 bits: the value's bits in the low half and the call's
// generation in the high half, written and read with relaxed atomics at
// agent scope, which keep it coherent across the chip's dies without a
// cache write-back.  A word carries its own validity, so no fence orders an
// exchange: a reader polls until every word it needs holds this call's
// generation, with all of its loads in flight before the first is used.
//
// Generations: the workspace counts the calls of the exchanging kernels run
// on it.  Where a launch of the same call precedes the exchanging one (the
// batched router before the batched gate/up kernel), that launch advances
// the count and the exchanging kernel takes the new count as g.  A single
// launch takes g = count + 1: every workgroup reads the count first and
// then raises its start flag to g, and workgroup 0 advances the count only
// at its very end and only after it has seen every start flag at g, so
// every workgroup of the call has read the same count.  A zeroed workspace
// starts at count 0 with every word at generation 0, never a call's.
//
// Every workgroup of such a launch must be resident at once; every wait is
// bounded: after XWAIT_TICKS a waiter stops, the call reports
// HFQ4_DEV_ERR_TIMEOUT, its outputs are undefined and the workspace must be
// zeroed again before its next use.
#pragma once
#include "hfq4_device.h"
#include "launch.h"

namespace hq {

constexpr uint64_t XWAIT_TICKS = 200000;   // 2 ms at 100 MHz

__device__ __forceinline__ void put_word(uint64_t* p, uint32_t bits, uint32_t g) {
  __hip_atomic_store(p, ((uint64_t)g << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_word(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll n tagged words at src[0..n) into dst (LDS) until all hold generation
// g, by the whole workgroup (at most PER_T words per thread, every load out
// before any is used).  Returns whether the wait expired.
template <int PER_T>
__device__ __forceinline__ bool gather_words(const uint64_t* src, int n, uint32_t g, float* dst) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const int nt = (int)blockDim.x;
  while (true) {
    uint64_t w[PER_T];
#pragma unroll
    for (int i = 0; i < PER_T; ++i) w[i] = get_word(src + min((int)threadIdx.x + nt * i, n - 1));
    int stale = 0;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int idx = (int)threadIdx.x + nt * i;
      if (idx < n) {
        stale |= (uint32_t)(w[i] >> 32) != g;
        dst[idx] = __uint_as_float((uint32_t)w[i]);
      }
    }
    const int any_stale = __syncthreads_or(stale);
    const int expired = __syncthreads_or(threadIdx.x == 0 &&
                                         __builtin_amdgcn_s_memrealtime() - t0 > XWAIT_TICKS);
    if (!any_stale) return false;
    if (expired) return true;
  }
}

// One wave: poll the start flags of workgroups 0 .. nwg - 1 (nwg <= XG_MAX)
// until all hold g.  Returns whether they did before the wait expired.
__device__ __forceinline__ bool start_flags_seen(const uint32_t* xflag, int nwg, uint32_t g) {
  const int lane = threadIdx.x & 63;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    uint32_t fw[XG_MAX / 64];
#pragma unroll
    for (int i = 0; i < XG_MAX / 64; ++i)   // clamped addresses: every load goes out at once
      fw[i] = __hip_atomic_load(const_cast<uint32_t*>(xflag) + min(lane + 64 * i, nwg - 1),
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool mine = true;
#pragma unroll
    for (int i = 0; i < XG_MAX / 64; ++i) mine &= fw[i] == g;
    if (__all(mine)) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 > XWAIT_TICKS) return false;
  }
}

}  // namespace hq
