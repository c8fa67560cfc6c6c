// Host (CPU) execution of HFQ4 experts: declarations shared by host_cpu.cpp
// and the C ABI.  Every pointer here is host memory.
#pragma once
#include <stdint.h>

namespace hq {

struct HostLayer {
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  int64_t E, d, F;
  int64_t stride_gate, stride_up, stride_down;
};

// Row kernels (set_host_kernel): the best the CPU has, or one forced.
enum { HOST_KERNEL_BEST = 0, HOST_KERNEL_AVX512 = 1, HOST_KERNEL_AVX2 = 2, HOST_KERNEL_SCALAR = 3 };
// Forces a row kernel for later calls (process-wide); false if the value is
// out of range or the CPU lacks the instructions.
bool set_host_kernel(int kernel);
// The row kernel calls use now (1..3).
int host_kernel_in_use();

// Threads a call uses when the caller passes 0.
int host_threads_default();

// y[b] = residual[b] + W x[b] for b < batch (W: HFQ4 rows of K).
void gemv_host(const uint8_t* W, int64_t rows, int64_t K, const float* x, int64_t ldx, int batch,
               const float* residual, int64_t ldr, float* y, int64_t ldy, int nthreads);

// The expert half of a layer for a token batch, on the host: for each
// token, y = residual + sum_j wts_j * down_e(SiLU(gate_e x) * (up_e x)), e =
// idx_j; an index outside [0, E) adds nothing and sets bit 1 of *err.
void expert_decode_host(const HostLayer& L, const float* x, int64_t ldx, int batch,
                        const int32_t* idx, const float* wts, int k, const float* residual,
                        float* y, int64_t ldy, int nthreads, uint32_t* err);

}  // namespace hq
