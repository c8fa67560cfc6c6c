// TurboQuant KV-vector codec on gfx950: encode f32 vectors of n = 64, 128 or
// 256 values into b-bit codes (b = 2, 3, 4 or 8) plus one f32 norm ratio,
// and decode them back.
//
// Page "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎", section "3.
// TurboQuant KV缓存压缩": each vector is normalised to unit L2 norm, rotated
// by a fast Walsh-Hadamard transform done with register-level lane swaps
// (no LDS and no barriers), quantised to Lloyd-Max centroids, and stored
// with the ratio of its norm to the norm of its reconstruction.  Readings
// (stated once, used by both kernels): the orthonormal Hadamard matrix in
// natural order, no random signs; the Lloyd-Max levels of the standard
// normal scaled by 1/sqrt(n), nearest level with ties to the lower one; the
// record is the codes packed LSB-first (code j at bits [j b, j b + b)) and
// then s = |v| / |c| as an f32.
//
// One wave per vector, n/64 consecutive values per lane: the butterflies of
// span h < n/64 stay in a lane, the others pair lane l with lane l ^
// (h / (n/64)) through a DPP quad permute or __shfl_xor; every output is the
// same sequence of exactly rounded adds and subtracts.  The level table is
// copied into LDS once per workgroup.  Both kernels are HBM streams: 4n
// bytes of f32 on one side, n b / 8 + 4 on the other.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hfq4_device.h"
#include "launch.h"

namespace hq {
namespace {

// value of lane l ^ m (m = 1, 2, ..., 32) in every lane: quad permutes by
// DPP for 1 and 2, the others by __shfl_xor (ds_bpermute: the LDS crossbar,
// no LDS memory and no barrier)
template <int M>
__device__ __forceinline__ float swap_lanes(float v) {
  if (M == 1) return dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if (M == 2) return dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  return __shfl_xor(v, M, 64);
}

// In-place orthonormal Walsh-Hadamard transform of the wave's n = 64 * EL
// values, lane l holding elements l*EL .. l*EL + EL - 1.
template <int EL>
__device__ __forceinline__ void fwht(float (&x)[EL], int lane) {
#pragma unroll
  for (int h = 1; h < EL; h <<= 1) {
#pragma unroll
    for (int e = 0; e < EL; ++e)
      if (!(e & h)) {
        const float a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
  }
  // spans >= EL: lanes l and l ^ m, m = h / EL
#define HQ_STAGE(M)                                            \
  {                                                            \
    const bool upper = (lane & (M)) != 0;                      \
    _Pragma("unroll") for (int e = 0; e < EL; ++e) {           \
      const float o = swap_lanes<M>(x[e]);                     \
      x[e] = upper ? o - x[e] : x[e] + o;                      \
    }                                                          \
  }
  HQ_STAGE(1) HQ_STAGE(2) HQ_STAGE(4) HQ_STAGE(8) HQ_STAGE(16) HQ_STAGE(32)
#undef HQ_STAGE
  const float inv = EL == 1 ? 0.125f : EL == 2 ? 0.08838834764831845f : 0.0625f;   // 1/sqrt(64 EL)
#pragma unroll
  for (int e = 0; e < EL; ++e) x[e] *= inv;
}

// wave sum of per-lane values in a fixed order
__device__ __forceinline__ float wsum(float v) { return wave_sum(v); }

template <int EL, int BITS>
__global__ void __launch_bounds__(256) turbo_encode_kernel(const float* __restrict__ v, int64_t count,
                                                           int64_t ldv, uint8_t* __restrict__ out,
                                                           TurboTable tab) {
  constexpr int N = 64 * EL, L = 1 << BITS;
  constexpr int REC = N * BITS / 8 + 4, CW = N * BITS / 32;   // record bytes, code words (<= 64)
  __shared__ uint32_t pk[4][CW];
  __shared__ float thr[L], cent[L];
  for (int i = threadIdx.x; i < L; i += blockDim.x) {
    cent[i] = tab.cent[i];
    thr[i] = i < L - 1 ? tab.thr[i] : INFINITY;
  }
  __syncthreads();
  const int wv = wave_id(), lane = threadIdx.x & 63;
  for (int64_t vec = (int64_t)blockIdx.x * 4 + wv; vec < count; vec += (int64_t)gridDim.x * 4) {
    float x[EL];
    const float* src = v + vec * ldv + lane * EL;
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = src[e];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    const float norm = __builtin_sqrtf(wsum(ss));
    const float inv = norm > 0.f ? 1.f / norm : 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] *= inv;
    fwht<EL>(x, lane);
    // nearest level: the number of thresholds strictly below r (binary search)
    uint32_t code[EL];
    float cc = 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      int lo = 0;
#pragma unroll
      for (int step = L / 2; step >= 1; step >>= 1)
        if (thr[lo + step - 1] < x[e]) lo += step;
      code[e] = norm > 0.f ? (uint32_t)lo : 0u;
      const float c = cent[code[e]];
      cc = __builtin_fmaf(c, c, cc);
    }
    const float cn = __builtin_sqrtf(wsum(cc));
    const float s = norm > 0.f ? norm / cn : 0.f;
    // pack: lane l's EL codes are bits [l EL BITS, (l+1) EL BITS) of the stream
    if (lane < CW) pk[wv][lane] = 0u;
    __builtin_amdgcn_wave_barrier();
    uint64_t chunk = 0;
#pragma unroll
    for (int e = 0; e < EL; ++e) chunk |= (uint64_t)code[e] << (e * BITS);
    const uint32_t bit0 = (uint32_t)lane * EL * BITS;
    const uint32_t w0 = bit0 >> 5, sh = bit0 & 31;
    const uint64_t placed = chunk << sh;
    atomicOr(&pk[wv][w0], (uint32_t)placed);
    if ((placed >> 32) != 0) atomicOr(&pk[wv][w0 + 1], (uint32_t)(placed >> 32));
    __builtin_amdgcn_wave_barrier();
    uint32_t* dst = reinterpret_cast<uint32_t*>(out + vec * REC);
    if (lane < CW) dst[lane] = pk[wv][lane];
    if (lane == 0) dst[CW] = __float_as_uint(s);
    __builtin_amdgcn_wave_barrier();
  }
}

template <int EL, int BITS>
__global__ void __launch_bounds__(256) turbo_decode_kernel(const uint8_t* __restrict__ in,
                                                           int64_t count, float* __restrict__ v,
                                                           int64_t ldv, TurboTable tab) {
  constexpr int N = 64 * EL, L = 1 << BITS;
  constexpr int REC = N * BITS / 8 + 4, CW = N * BITS / 32;   // record bytes, code words (<= 64)
  __shared__ float cent[L];
  for (int i = threadIdx.x; i < L; i += blockDim.x) cent[i] = tab.cent[i];
  __syncthreads();
  const int wv = wave_id(), lane = threadIdx.x & 63;
  for (int64_t vec = (int64_t)blockIdx.x * 4 + wv; vec < count; vec += (int64_t)gridDim.x * 4) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(in + vec * REC);
    const uint32_t mine = lane < CW ? src[lane] : 0u;
    const float s = __uint_as_float(src[CW]);
    const uint32_t bit0 = (uint32_t)lane * EL * BITS;
    const int w0 = (int)(bit0 >> 5), sh = (int)(bit0 & 31);
    const uint32_t lo = __shfl(mine, w0, 64), hi = __shfl(mine, min(w0 + 1, CW - 1), 64);
    const uint64_t chunk = (((uint64_t)hi << 32) | lo) >> sh;
    float x[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = cent[(chunk >> (e * BITS)) & ((1u << BITS) - 1)];
    fwht<EL>(x, lane);
    float* dst = v + vec * ldv + lane * EL;
#pragma unroll
    for (int e = 0; e < EL; ++e) dst[e] = s * x[e];
  }
}

template <int EL>
int launch_turbo_el(bool enc, const void* src, int64_t count, int64_t ld, void* dst, int bits,
                    const TurboTable& tab, hipStream_t s) {
  int64_t blocks = (count + 3) / 4;
  if (blocks > 8192) blocks = 8192;
#define HQ_T(B)                                                                                  \
  if (bits == B) {                                                                               \
    if (enc)                                                                                     \
      hipLaunchKernelGGL((turbo_encode_kernel<EL, B>), dim3((unsigned)blocks), dim3(256), 0, s, \
                         static_cast<const float*>(src), count, ld, static_cast<uint8_t*>(dst), tab); \
    else                                                                                         \
      hipLaunchKernelGGL((turbo_decode_kernel<EL, B>), dim3((unsigned)blocks), dim3(256), 0, s, \
                         static_cast<const uint8_t*>(src), count, static_cast<float*>(dst), ld, tab); \
    return (int)hipGetLastError();                                                               \
  }
  HQ_T(2) HQ_T(3) HQ_T(4) HQ_T(8)
#undef HQ_T
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_turbo(bool encode, const void* src, int64_t count, int n, int64_t ld, void* dst,
                 int bits, const TurboTable& tab, hipStream_t s) {
  if (count == 0) return 0;
  if (n == 64) return launch_turbo_el<1>(encode, src, count, ld, dst, bits, tab, s);
  if (n == 128) return launch_turbo_el<2>(encode, src, count, ld, dst, bits, tab, s);
  if (n == 256) return launch_turbo_el<4>(encode, src, count, ld, dst, bits, tab, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace hq
