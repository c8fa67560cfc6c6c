// hfq4_pack: f32 rows -> canonical HFQ4 bytes, one wave per 256-weight block.
//
// Format: page "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎", section
// "2. HFQ量化格式与GEMV优化" (136-byte block: f32 scale, f32 zero point,
// 128 code bytes).  Quantizer (a reading; the page gives only the fields):
// zero = block min, scale = f32(f32(max - min) / 15), q = clamp(rint(f32(
// f32(w - zero) / scale)), 0, 15), ties to even; scale 0 => all codes 0.
// -0.0 and +0.0 compare equal, so which zero a min reduction returns depends
// on its order; the zero field is the minimum plus +0.0, which is +0.0 for
// either zero and the minimum itself otherwise, so the bytes never depend
// on the reduction order.
// The f32 subtract and the correctly rounded f32 divide make every code
// decision identical to a host f32 implementation of the same definition.
#include "hfq4_device.h"
#include "launch.h"

namespace hq {

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fminf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__global__ void __launch_bounds__(256) pack_kernel(const float* __restrict__ w, int64_t rows,
                                                   int64_t K, int64_t ldw, uint8_t* __restrict__ out,
                                                   int32_t* bad) {
  const int lane = threadIdx.x & 63;
  const int64_t nb = (K + BLK - 1) / BLK;
  const int64_t total = rows * nb;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_id();
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t blk = wave; blk < total; blk += nwaves) {
    const int64_t r = blk / nb, b = blk - r * nb;
    const float* src = w + r * ldw + b * BLK;
    const int64_t nvalid64 = K - b * BLK;
    const int nvalid = nvalid64 < BLK ? (int)nvalid64 : BLK;
    float v[4];
    bool valid[4];
    int finite = 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      valid[i] = e < nvalid;
      v[i] = valid[i] ? src[e] : 0.f;
      finite &= (!valid[i]) || __builtin_isfinite(v[i]);
    }
    float lmin = INFINITY, lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (valid[i]) {
        lmin = fminf(lmin, v[i]);
        lmax = fmaxf(lmax, v[i]);
      }
    }
    const bool all_finite = __all(finite);
    const float mn = wave_min(lmin), mx = wave_max(lmax);
    const float range = mx - mn;
    uint8_t* dst = out + blk * BLK_BYTES;
    if (!all_finite || !__builtin_isfinite(range)) {
      // rejected block: all-zero bytes, counted once
      if (lane < 34) reinterpret_cast<uint32_t*>(dst)[lane] = 0u;
      if (lane == 0 && bad) atomicAdd(bad, 1);
      continue;
    }
    const float scale = range / 15.0f;   // correctly rounded f32 divide
    const float zero = mn + 0.0f;        // -0.0 -> +0.0 (not folded: IEEE signed zeros)
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float t = 0.f;
      if (valid[i] && scale != 0.f) t = rintf((v[i] - zero) / scale);
      t = fminf(fmaxf(t, 0.f), 15.f);
      q[i] = valid[i] ? (uint32_t)t : 0u;
    }
    const uint32_t two = (q[0] | (q[1] << 4)) | ((q[2] | (q[3] << 4)) << 8);
    reinterpret_cast<uint16_t*>(dst + 8)[lane] = (uint16_t)two;
    if (lane == 0) {
      reinterpret_cast<float*>(dst)[0] = scale;
      reinterpret_cast<float*>(dst)[1] = zero;
    }
  }
}

int launch_pack(const float* w, int64_t rows, int64_t K, int64_t ldw, void* out, int32_t* bad,
                hipStream_t s) {
  const int64_t total = rows * ((K + BLK - 1) / BLK);
  if (total == 0) return 0;
  int64_t blocks = (total + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, rows, K, ldw,
                     static_cast<uint8_t*>(out), bad);
  return (int)hipGetLastError();
}

}  // namespace hq
