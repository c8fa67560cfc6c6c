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

// ---------------------------------------------------------------- streaming read

// Every lane reads 16-byte chunks, grid-strided, four in flight; one sum per
// workgroup is written so the loads stay live.
__global__ void __launch_bounds__(256) read_kernel(const uint4* __restrict__ p, size_t n16,
                                                   uint32_t* sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ b.y ^ c.z ^ d.w;
  }
  for (; i < n16; i += stride) acc ^= p[i].x;
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

int probe_read(const void* p, size_t bytes, int grid, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(p),
                     bytes / 16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
