// Latency and bandwidth probes behind the decode path's floor model
// (libhfq4probe.so; measurement only, not part of the decode library).
//
// Every kernel here is bounded: loops run a fixed number of steps and every
// wait on another workgroup gives up after a fixed number of polls (the
// result then reports the timeout instead of a latency).  Times come from
// s_memrealtime (100 MHz) inside the kernels or from HIP events around
// launches on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xFu;
}

// ---------------------------------------------------------------- pointer chase

// One lane follows next[] for `hops` dependent loads: the average time per
// hop is the load-to-use latency of whatever level of the memory hierarchy
// the chain's footprint falls in.  out[0] = elapsed ticks, out[1] = the
// final index (keeps the chain live).
__global__ void chase_kernel(const uint32_t* __restrict__ next, uint32_t start, int hops,
                             uint64_t* out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  uint32_t i = start;
  // the first part of the chain is not timed (instruction cache, first TLB
  // entries)
  for (int h = 0; h < 64; ++h) i = next[i];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const uint64_t t0 = now();
  for (int h = 0; h < hops; ++h) i = next[i];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const uint64_t t1 = now();
  out[0] = t1 - t0;
  out[1] = i;
}

// ---------------------------------------------------------------- empty kernels

__global__ void empty_kernel(uint32_t* sink) {
  if (sink && threadIdx.x == 0 && blockIdx.x == 0x7fffffff) sink[0] = 1u;   // never taken
}

// One link of a chain of dependent launches: every thread reads the value
// the previous launch wrote at its index and writes its own.  Plain pointer
// arguments, so that a build with the kernel arguments preloaded into
// scalar registers can preload them.
__global__ void chain_kernel(const float* __restrict__ in, float* __restrict__ out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = in[i] + 1.f;
}

// ---------------------------------------------------------------- cross-XCD flags

// Ping-pong between workgroup 0 and workgroup `partner` (both single-wave;
// every other workgroup exits at once).  Round r: the pinger stores r+1 to
// its flag, the ponger waits for it and answers with r+1 on its own flag,
// the pinger waits for the answer.  Flags are read and written with relaxed
// atomics at agent scope (coherent across the chip's dies); with `release`
// the pinger also writes `payload_words` words of data before its flag with
// a release store, and the ponger reads them after an acquire load (the
// message-passing pattern with its fences).  out[0..1] = elapsed ticks of
// the two sides, out[2..3] = their die ids, out[4] = 1 if a wait timed out.
__global__ void pingpong_kernel(uint32_t* flags, uint32_t* payload, int payload_words, int rounds,
                                int partner, int release, uint64_t* out) {
  const bool ping = blockIdx.x == 0;
  if (!ping && (int)blockIdx.x != partner) return;
  const int lane = threadIdx.x;
  uint32_t* mine = flags + (ping ? 0 : 32);      // separate 128-byte lines
  uint32_t* theirs = flags + (ping ? 32 : 0);
  const int kMaxPolls = 1 << 20;
  bool timeout = false;
  uint32_t sink = 0;
  const uint64_t t0 = now();
  for (int r = 0; r < rounds && !timeout; ++r) {
    const uint32_t v = (uint32_t)r + 1u;
    if (ping) {
      if (release) {
        for (int w = lane; w < payload_words; w += 64) payload[w] = v ^ (uint32_t)w;
        __syncthreads();
        if (lane == 0) __hip_atomic_store(mine, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else if (lane == 0) {
        __hip_atomic_store(mine, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // wait for the other side's flag (ping waits for the answer to round r,
    // pong for round r's ping)
    int polls = 0;
    uint32_t seen = 0;
    if (lane == 0) {
      if (release && !ping) {
        while ((seen = __hip_atomic_load(theirs, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)) != v &&
               ++polls < kMaxPolls) {
        }
      } else {
        while ((seen = __hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != v &&
               ++polls < kMaxPolls) {
        }
      }
    }
    seen = __builtin_amdgcn_readfirstlane(seen);
    timeout = seen != v;
    if (!ping && !timeout) {
      if (release)
        for (int w = lane; w < payload_words; w += 64) sink += payload[w];
      if (lane == 0) __hip_atomic_store(mine, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const uint64_t t1 = now();
  if (lane == 0) {
    out[ping ? 0 : 1] = t1 - t0;
    out[ping ? 2 : 3] = xcc_id();
    if (timeout) out[4] = 1;
  }
  if (sink == 0xFFFFFFFFu && lane == 0) out[5] = sink;   // keeps the payload reads
}

// ---------------------------------------------------------------- boundary + first read

// Producer: every workgroup writes one 4-byte value (like a router logit)
// and stamps its end time.
__global__ void produce_kernel(float* vals, uint64_t* stamps) {
  if (threadIdx.x == 0) {
    vals[blockIdx.x] = (float)blockIdx.x;
    stamps[blockIdx.x] = now();
  }
}

// Consumer (the next launch on the stream): every workgroup stamps its
// start, reads all `n` values (as the expert kernel reads the logits), and
// stamps the arrival of the data.  stamps[n + wg] = start, [2n + wg] = data
// arrived, [3n + wg] = die id.
__global__ void consume_kernel(const float* vals, int n, uint64_t* stamps, float* sink) {
  const uint64_t t0 = now();
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s += vals[i];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const uint64_t t1 = now();
  if (threadIdx.x == 0) {
    stamps[n + blockIdx.x] = t0;
    stamps[2 * n + blockIdx.x] = t1;
    stamps[3 * n + blockIdx.x] = xcc_id();
  }
  if (s == -1.f) sink[0] = s;   // never true for these values; keeps the loads
}

// ---------------------------------------------------------------- all-to-all exchange

// Every workgroup publishes `per_wg` 64-bit words (value, tag) with relaxed
// agent-scope atomic stores, then polls all nwg * per_wg words until every
// tag is this run's, up to a bounded number of rounds -- the data exchange
// a single-launch layer would need between its phases (router logits: one
// word per workgroup; h: 16 per workgroup).  With `flags`, a workgroup also
// raises a tagged per-workgroup flag after its words and the pollers first
// wait for all flags, then read the words once (re-reading any stale one).
// stamps[wg] = publish time, stamps[nwg + wg] = all data seen, stamps[2 nwg
// + wg] = poll rounds, stamps[3 nwg + wg] = 1 on timeout.
__global__ void __launch_bounds__(256) exchange_kernel(uint64_t* words, uint32_t* flagw, int per_wg,
                                                       uint32_t tag, int flags, uint64_t* stamps,
                                                       int replicas, int stagger) {
  const int nwg = gridDim.x, wg = blockIdx.x, t = threadIdx.x;
  const int total = nwg * per_wg;
  // each word goes to `replicas` copies; a reader polls copy wg % replicas
  // (with round-robin placement of workgroups on dies, copy = die for 8)
  for (int i = t; i < per_wg * replicas; i += blockDim.x) {
    const int r = i / per_wg, j = i - r * per_wg;
    const uint64_t w = ((uint64_t)tag << 32) | (uint32_t)(wg * per_wg + j);
    __hip_atomic_store(words + (size_t)r * total + wg * per_wg + j, w, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  const uint64_t* mine = words + (size_t)(wg % replicas) * total;
  const int rot = stagger ? (wg * 64) % total : 0;   // readers start at different words
  __syncthreads();
  if (flags && t == 0) __hip_atomic_store(flagw + wg, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t t0 = now();
  int rounds = 0, missing = 0;
  const int kMaxRounds = 100000;
  if (flags) {
    do {
      int miss = 0;
      for (int i = t; i < nwg; i += blockDim.x)
        miss |= __hip_atomic_load(flagw + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag;
      missing = __syncthreads_or(miss);
      ++rounds;
    } while (missing && rounds < kMaxRounds);
  }
  do {
    int miss = 0;
    uint64_t w[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = t + u * 256;
      int j = i + rot;
      j = j >= total ? j - total : j;
      w[u] = __hip_atomic_load(const_cast<uint64_t*>(mine) + (i < total ? j : 0), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) miss |= (t + u * 256 < total) && (uint32_t)(w[u] >> 32) != tag;
    missing = __syncthreads_or(miss);
    ++rounds;
  } while (missing && rounds < kMaxRounds);
  const uint64_t t1 = now();
  if (t == 0) {
    stamps[wg] = t0;
    stamps[nwg + wg] = t1;
    stamps[2 * nwg + wg] = rounds;
    stamps[3 * nwg + wg] = missing ? 1 : 0;
  }
}

// ---------------------------------------------------------------- spin

// One wave that keeps the device busy for `ticks` (100 MHz) and exits: put
// in front of a timed region, it lets the host enqueue the region's work
// before the device reaches it.
__global__ void spin_kernel(uint64_t ticks) {
  const uint64_t t0 = now();
  while (now() - t0 < ticks) __builtin_amdgcn_s_sleep(2);
}

// ---------------------------------------------------------------- streaming read

// Every lane reads 16-byte chunks, eight in flight; each workgroup walks a
// contiguous slice of the buffer (chunks of 8 x 4 KiB per step), and one
// value per workgroup is written so the loads stay live.
__global__ void __launch_bounds__(256) read_kernel(const uint4* __restrict__ p, size_t n16,
                                                   uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].w;
  }
  for (; i < hi; i += 256) acc ^= p[i].x;
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// All launches go on `stream`; results are valid once it reaches them.
int probe_chase(const uint32_t* next, uint32_t start, int hops, uint64_t* out, hipStream_t s) {
  hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(64), 0, s, next, start, hops, out);
  return (int)hipGetLastError();
}

int probe_empty(int grid, int block, hipStream_t s) {
  hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(block), 0, s, (uint32_t*)nullptr);
  return (int)hipGetLastError();
}

int probe_chain(const float* in, float* out, int n, hipStream_t s) {
  if (n < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(chain_kernel, dim3((n + 63) / 64), dim3(64), 0, s, in, out, n);
  return (int)hipGetLastError();
}

int probe_pingpong(uint32_t* flags, uint32_t* payload, int payload_words, int rounds, int partner,
                   int release, uint64_t* out, hipStream_t s) {
  if (partner < 1 || partner > 4095 || rounds < 1 || payload_words < 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(pingpong_kernel, dim3(partner + 1), dim3(64), 0, s, flags, payload,
                     payload_words, rounds, partner, release, out);
  return (int)hipGetLastError();
}

int probe_produce(float* vals, int n, uint64_t* stamps, hipStream_t s) {
  hipLaunchKernelGGL(produce_kernel, dim3(n), dim3(64), 0, s, vals, stamps);
  return (int)hipGetLastError();
}

int probe_consume(const float* vals, int n, uint64_t* stamps, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(consume_kernel, dim3(n), dim3(64), 0, s, vals, n, stamps, sink);
  return (int)hipGetLastError();
}

int probe_exchange(uint64_t* words, uint32_t* flagw, int nwg, int per_wg, uint32_t tag, int flags,
                   uint64_t* stamps, int replicas, int stagger, hipStream_t s) {
  if (nwg < 1 || nwg > 1024 || per_wg < 1 || nwg * per_wg > 4096 || replicas < 1 || replicas > 64)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(exchange_kernel, dim3(nwg), dim3(256), 0, s, words, flagw, per_wg, tag, flags,
                     stamps, replicas, stagger);
  return (int)hipGetLastError();
}

int probe_spin(uint64_t ticks, hipStream_t s) {
  if (ticks > 10000000ull) return (int)hipErrorInvalidValue;   // at most 0.1 s
  hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, s, ticks);
  return (int)hipGetLastError();
}

int probe_read(const void* p, size_t bytes, int grid, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(p),
                     bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
