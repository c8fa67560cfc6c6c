// HFQ4 expert execution on the host CPU (x86-64: AVX-512, or AVX2 + FMA,
// with a portable fallback): the other side of host-resident experts.
//
// Host-resident experts can be computed where they live instead of being
// read over PCIe by a GPU kernel: the hipfire expert-offload explainer,
// section "PCIe 直通", times the PCIe link against a CPU GEMV at load and
// runs on the CPU only when that is at least 15% faster (its "D2 measured
// default"); the Strata user report, sections "1. Strata 是什么" and "2.
// 硬件配置", runs the experts that miss its VRAM cache on the CPU with AVX-2
// kernels.  Here the same HFQ4 arithmetic as the GPU path, in f32, with the
// activation de-interleaved once per call so that the low nibbles of a run
// of code bytes meet the even elements and the high nibbles the odd ones
// (no shuffles of x in the inner loops).  Two row kernels:
//   * AVX-512: each block's 16 dequantized values zero + scale q are a
//     register table that the nibbles index (a lane permute), products
//     summed across the row;
//   * AVX2 (and the portable one): per 256-weight block
//     sum_i (zero + scale q_i) x_i = zero * sum_i x_i + scale * sum_i q_i x_i.
// The best the CPU has runs unless a diagnostic call forces another.
//
// Threads: a small pool of host threads, created on first use and kept
// until the process ends, takes contiguous row ranges; every output element
// is summed by one thread in a fixed order, so results do not depend on the
// thread count.
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#if defined(__x86_64__)
#include <immintrin.h>
#endif
#if defined(__linux__)
#include <sched.h>
#endif

#include "host_cpu.h"

namespace hq {
namespace {

constexpr int BLKW = 256;      // weights per block
constexpr int BLKB = 136;      // bytes per block
constexpr int HALF = 128;      // code bytes per block

// ------------------------------------------------------------ thread pool

class Pool {
 public:
  // Run fn(t, n) for t = 0..n-1, the caller taking t = 0; returns when all
  // have finished.  Calls are serialised.
  void run(int n, const std::function<void(int, int)>& fn) {
    std::lock_guard<std::mutex> call(call_mu_);
    if (n <= 1) {
      fn(0, 1);
      return;
    }
    grow(n - 1);
    {
      std::lock_guard<std::mutex> lk(mu_);
      job_ = &fn;
      njob_ = n;
      pending_.store(n - 1);
      epoch_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
    fn(0, n);
    // the workers of this call spin briefly before sleeping, so a decode's
    // back-to-back calls see them awake
    while (pending_.load(std::memory_order_acquire) != 0) {
#if defined(__x86_64__)
      _mm_pause();
#endif
    }
  }

 private:
  void grow(int want) {
    while ((int)threads_.size() < want) {
      const int id = (int)threads_.size() + 1;
      threads_.emplace_back([this, id] { worker(id); });
      threads_.back().detach();
    }
  }
  void worker(int id) {
    uint64_t seen = 0;
    for (;;) {
      const std::function<void(int, int)>* job = nullptr;
      int n = 0;
      {
        // spin on the epoch for a while, then sleep
        for (int s = 0; s < 20000; ++s) {
          if (epoch_.load(std::memory_order_acquire) != seen) break;
#if defined(__x86_64__)
          _mm_pause();
#endif
        }
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return epoch_.load(std::memory_order_acquire) != seen; });
        seen = epoch_.load(std::memory_order_acquire);
        job = job_;
        n = njob_;
      }
      if (id < n) {
        (*job)(id, n);
        pending_.fetch_sub(1, std::memory_order_acq_rel);
      }
    }
  }
  std::mutex call_mu_, mu_;
  std::condition_variable cv_;
  std::vector<std::thread> threads_;
  const std::function<void(int, int)>* job_ = nullptr;
  int njob_ = 0;
  std::atomic<uint64_t> epoch_{0};
  std::atomic<int> pending_{0};
};

Pool& pool() {
  static Pool* p = new Pool();   // lives until the process ends
  return *p;
}

// ------------------------------------------------------------ activations

// One activation vector in the layout the row kernel reads: per block b,
// xe[b][j] = x[256b + 2j], xo[b][j] = x[256b + 2j + 1] (0 past K), and the
// block sum sx[b] of the valid elements.
struct XPrep {
  std::vector<float> xe, xo, sx;
  int nb = 0;
  void build(const float* x, int64_t K) {
    nb = (int)((K + BLKW - 1) / BLKW);
    xe.assign((size_t)nb * HALF, 0.f);
    xo.assign((size_t)nb * HALF, 0.f);
    sx.assign(nb, 0.f);
    for (int b = 0; b < nb; ++b) {
      float s = 0.f;
      for (int j = 0; j < HALF; ++j) {
        const int64_t i0 = (int64_t)b * BLKW + 2 * j, i1 = i0 + 1;
        const float a = i0 < K ? x[i0] : 0.f, c = i1 < K ? x[i1] : 0.f;
        xe[(size_t)b * HALF + j] = a;
        xo[(size_t)b * HALF + j] = c;
        s += a + c;
      }
      sx[b] = s;
    }
  }
};

// sum_j q_lo[j] * xe[j] + q_hi[j] * xo[j] over one block's 128 code bytes.
float block_dot_scalar(const uint8_t* codes, const float* xe, const float* xo) {
  float a = 0.f, c = 0.f;
  for (int j = 0; j < HALF; ++j) {
    a = std::fma((float)(codes[j] & 15), xe[j], a);
    c = std::fma((float)(codes[j] >> 4), xo[j], c);
  }
  return a + c;
}

#if defined(__x86_64__)
__attribute__((target("avx2,fma"))) float block_dot_avx2(const uint8_t* codes, const float* xe,
                                                         const float* xo) {
  const __m256i m15 = _mm256_set1_epi32(15);
  __m256 a0 = _mm256_setzero_ps(), a1 = _mm256_setzero_ps();
  __m256 c0 = _mm256_setzero_ps(), c1 = _mm256_setzero_ps();
  for (int j = 0; j < HALF; j += 16) {
    const __m256i v0 = _mm256_cvtepu8_epi32(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(codes + j)));
    const __m256i v1 =
        _mm256_cvtepu8_epi32(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(codes + j + 8)));
    const __m256 lo0 = _mm256_cvtepi32_ps(_mm256_and_si256(v0, m15));
    const __m256 hi0 = _mm256_cvtepi32_ps(_mm256_srli_epi32(v0, 4));
    const __m256 lo1 = _mm256_cvtepi32_ps(_mm256_and_si256(v1, m15));
    const __m256 hi1 = _mm256_cvtepi32_ps(_mm256_srli_epi32(v1, 4));
    a0 = _mm256_fmadd_ps(lo0, _mm256_loadu_ps(xe + j), a0);
    c0 = _mm256_fmadd_ps(hi0, _mm256_loadu_ps(xo + j), c0);
    a1 = _mm256_fmadd_ps(lo1, _mm256_loadu_ps(xe + j + 8), a1);
    c1 = _mm256_fmadd_ps(hi1, _mm256_loadu_ps(xo + j + 8), c1);
  }
  const __m256 t = _mm256_add_ps(_mm256_add_ps(a0, a1), _mm256_add_ps(c0, c1));
  __m128 s = _mm_add_ps(_mm256_castps256_ps128(t), _mm256_extractf128_ps(t, 1));
  s = _mm_add_ps(s, _mm_movehl_ps(s, s));
  s = _mm_add_ss(s, _mm_shuffle_ps(s, s, 1));
  return _mm_cvtss_f32(s);
}
#endif

using BlockDot = float (*)(const uint8_t*, const float*, const float*);

// Rows [r0, r1) of y = W x (+ residual) for one prepared vector, one block
// dot product at a time: per block scale * sum q x + zero * sum x.
void rows_dot_blocks(BlockDot dot, const uint8_t* W, int64_t r0, int64_t r1, int nb,
                     const XPrep& xp, const float* res, float* y) {
  const int64_t rowb = (int64_t)nb * BLKB;
  for (int64_t r = r0; r < r1; ++r) {
    const uint8_t* row = W + r * rowb;
    float acc = 0.f;
    for (int b = 0; b < nb; ++b) {
      const uint8_t* blk = row + (int64_t)b * BLKB;
      float scale, zero;
      std::memcpy(&scale, blk, 4);
      std::memcpy(&zero, blk + 4, 4);
      const float qd = dot(blk + 8, &xp.xe[(size_t)b * HALF], &xp.xo[(size_t)b * HALF]);
      acc += std::fma(scale, qd, zero * xp.sx[b]);
    }
    y[r] = (res ? res[r] : 0.f) + acc;
  }
}

#if defined(__x86_64__)
// AVX-512 rows: per block a 16-entry table of the block's dequantized values
// zero + scale * q (one f32 fma each, the format's definition), looked up by
// the code nibbles with a lane permute (its index is the low 4 bits of each
// 32-bit lane, so the low nibble needs no mask), and the products
// accumulated in four vectors across the whole row; one horizontal sum per
// row.  A permute pair covers 16 code bytes = 32 weights.
__attribute__((target("avx512f"))) void rows_dot_avx512(const uint8_t* W, int64_t r0, int64_t r1,
                                                        int nb, const XPrep& xp, const float* res,
                                                        float* y) {
  const __m512 iota = _mm512_setr_ps(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  const int64_t rowb = (int64_t)nb * BLKB;
  for (int64_t r = r0; r < r1; ++r) {
    const uint8_t* row = W + r * rowb;
    __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps();
    __m512 a2 = _mm512_setzero_ps(), a3 = _mm512_setzero_ps();
    for (int b = 0; b < nb; ++b) {
      const uint8_t* blk = row + (int64_t)b * BLKB;
      float scale, zero;
      std::memcpy(&scale, blk, 4);
      std::memcpy(&zero, blk + 4, 4);
      const __m512 tab = _mm512_fmadd_ps(iota, _mm512_set1_ps(scale), _mm512_set1_ps(zero));
      const uint8_t* codes = blk + 8;
      const float* xe = &xp.xe[(size_t)b * HALF];
      const float* xo = &xp.xo[(size_t)b * HALF];
      for (int j = 0; j < HALF; j += 32) {
        const __m512i v0 =
            _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + j)));
        const __m512i v1 =
            _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + j + 16)));
        a0 = _mm512_fmadd_ps(_mm512_permutexvar_ps(v0, tab), _mm512_loadu_ps(xe + j), a0);
        a1 = _mm512_fmadd_ps(_mm512_permutexvar_ps(_mm512_srli_epi32(v0, 4), tab),
                             _mm512_loadu_ps(xo + j), a1);
        a2 = _mm512_fmadd_ps(_mm512_permutexvar_ps(v1, tab), _mm512_loadu_ps(xe + j + 16), a2);
        a3 = _mm512_fmadd_ps(_mm512_permutexvar_ps(_mm512_srli_epi32(v1, 4), tab),
                             _mm512_loadu_ps(xo + j + 16), a3);
      }
    }
    const float acc =
        _mm512_reduce_add_ps(_mm512_add_ps(_mm512_add_ps(a0, a1), _mm512_add_ps(a2, a3)));
    y[r] = (res ? res[r] : 0.f) + acc;
  }
}
#endif

bool cpu_has(int kernel) {
  if (kernel == HOST_KERNEL_SCALAR) return true;
#if defined(__x86_64__)
  __builtin_cpu_init();
  if (kernel == HOST_KERNEL_AVX512) return __builtin_cpu_supports("avx512f");
  if (kernel == HOST_KERNEL_AVX2)
    return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
#endif
  return false;
}

int best_kernel() {
  static const int k = cpu_has(HOST_KERNEL_AVX512) ? HOST_KERNEL_AVX512
                       : cpu_has(HOST_KERNEL_AVX2) ? HOST_KERNEL_AVX2
                                                   : HOST_KERNEL_SCALAR;
  return k;
}

std::atomic<int> g_host_kernel{HOST_KERNEL_BEST};

void rows_dot(const uint8_t* W, int64_t r0, int64_t r1, int nb, const XPrep& xp, const float* res,
              float* y) {
  int kern = g_host_kernel.load(std::memory_order_relaxed);
  if (kern == HOST_KERNEL_BEST) kern = best_kernel();
#if defined(__x86_64__)
  if (kern == HOST_KERNEL_AVX512) return rows_dot_avx512(W, r0, r1, nb, xp, res, y);
  if (kern == HOST_KERNEL_AVX2) return rows_dot_blocks(block_dot_avx2, W, r0, r1, nb, xp, res, y);
#endif
  rows_dot_blocks(block_dot_scalar, W, r0, r1, nb, xp, res, y);
}

inline void split(int64_t n, int t, int nt, int64_t& lo, int64_t& hi) {
  lo = n * t / nt;
  hi = n * (t + 1) / nt;
}

inline float silu_mul_host(float g, float u) { return g / (1.f + std::exp(-g)) * u; }

}  // namespace

bool set_host_kernel(int kernel) {
  if (kernel < HOST_KERNEL_BEST || kernel > HOST_KERNEL_SCALAR) return false;
  if (kernel != HOST_KERNEL_BEST && !cpu_has(kernel)) return false;
  g_host_kernel.store(kernel, std::memory_order_relaxed);
  return true;
}

int host_kernel_in_use() {
  const int k = g_host_kernel.load(std::memory_order_relaxed);
  return k == HOST_KERNEL_BEST ? best_kernel() : k;
}

int host_threads_default() {
  // the CPUs this process may run on (a container or a scheduler may grant
  // far fewer than the machine has), at most OMP_NUM_THREADS when that is
  // set, at most 64: more threads than CPUs would leave spinning workers
  // competing with the ones that compute
  int n = 0;
#if defined(__linux__)
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof set, &set) == 0) n = CPU_COUNT(&set);
#endif
  if (n <= 0) n = (int)std::thread::hardware_concurrency();
  if (const char* e = std::getenv("OMP_NUM_THREADS")) {
    const int m = std::atoi(e);
    if (m > 0 && m < n) n = m;
  }
  return n < 1 ? 1 : (n > 64 ? 64 : n);
}

void gemv_host(const uint8_t* W, int64_t rows, int64_t K, const float* x, int64_t ldx, int batch,
               const float* residual, int64_t ldr, float* y, int64_t ldy, int nthreads) {
  std::vector<XPrep> xp(batch);
  for (int b = 0; b < batch; ++b) xp[b].build(x + b * ldx, K);
  const int nb = xp[0].nb;
  const int nt = (int)std::min<int64_t>(nthreads, std::max<int64_t>(1, rows / 16));
  pool().run(nt, [&](int t, int n) {
    int64_t lo, hi;
    split(rows, t, n, lo, hi);
    for (int b = 0; b < batch; ++b)
      rows_dot(W, lo, hi, nb, xp[b], residual ? residual + b * ldr : nullptr, y + b * ldy);
  });
}

void expert_decode_host(const HostLayer& L, const float* x, int64_t ldx, int batch,
                        const int32_t* idx, const float* wts, int k, const float* residual,
                        float* y, int64_t ldy, int nthreads, uint32_t* err) {
  const int64_t d = L.d, F = L.F;
  const int nbd = (int)((d + BLKW - 1) / BLKW), nbf = (int)((F + BLKW - 1) / BLKW);
  std::vector<float> h((size_t)k * F);
  std::vector<float> yslot((size_t)k * d);
  for (int b = 0; b < batch; ++b) {
    XPrep xp;
    xp.build(x + b * ldx, d);
    std::vector<int> ex(k);
    for (int j = 0; j < k; ++j) {
      const int e = idx[b * k + j];
      ex[j] = (e >= 0 && e < L.E) ? e : -1;
      if (ex[j] < 0 && err) *err |= 1u;   // HFQ4_DEV_ERR_INDEX: the slot adds nothing
    }
    // gate/up of every slot: 2 k F rows over the threads
    std::vector<float> gu((size_t)2 * k * F);
    const int64_t nrow_gu = 2 * (int64_t)k * F;
    const int nt = (int)std::min<int64_t>(nthreads, std::max<int64_t>(1, nrow_gu / 32));
    pool().run(nt, [&](int t, int n) {
      int64_t lo, hi;
      split(nrow_gu, t, n, lo, hi);
      for (int64_t r = lo; r < hi; ++r) {
        const int64_t j = r / (2 * F), rem = r - j * 2 * F;
        const bool up = rem >= F;
        const int64_t f = up ? rem - F : rem;
        if (ex[j] < 0) {
          gu[r] = 0.f;
          continue;
        }
        const uint8_t* W = (up ? L.up + (int64_t)ex[j] * L.stride_up
                               : L.gate + (int64_t)ex[j] * L.stride_gate);
        rows_dot(W, f, f + 1, nbd, xp, nullptr, &gu[r] - f);
      }
    });
    for (int j = 0; j < k; ++j)
      for (int64_t f = 0; f < F; ++f)
        h[(size_t)j * F + f] =
            silu_mul_host(gu[(size_t)2 * j * F + f], gu[(size_t)2 * j * F + F + f]);
    // down of every slot, then the weighted sum in slot order per row
    std::vector<XPrep> hp(k);
    for (int j = 0; j < k; ++j) hp[j].build(&h[(size_t)j * F], F);
    const int nt2 = (int)std::min<int64_t>(nthreads, std::max<int64_t>(1, d / 16));
    pool().run(nt2, [&](int t, int n) {
      int64_t lo, hi;
      split(d, t, n, lo, hi);
      for (int j = 0; j < k; ++j) {
        if (ex[j] < 0) continue;
        const uint8_t* W = L.down + (int64_t)ex[j] * L.stride_down;
        rows_dot(W, lo, hi, nbf, hp[j], nullptr, &yslot[(size_t)j * d]);
      }
      for (int64_t r = lo; r < hi; ++r) {
        float acc = residual ? residual[b * ldy + r] : 0.f;
        for (int j = 0; j < k; ++j)
          if (ex[j] >= 0) acc = std::fma(wts[b * k + j], yslot[(size_t)j * d + r], acc);
        y[b * ldy + r] = acc;
      }
    });
  }
}

}  // namespace hq
