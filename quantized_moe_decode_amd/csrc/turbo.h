// TurboQuant codec: the level table the kernels take (host-side helpers;
// the launcher is declared in launch.h).
#pragma once
#include <stdint.h>

namespace hq {

// Levels of one (n, bits) codec: cent[0 .. 2^bits) ascending (already
// scaled by 1/sqrt(n)) and thr[m] = the midpoint of cent[m], cent[m+1].
struct TurboTable {
  float cent[256];
  float thr[255];
  // Bucket index of a value r for the nearest-level search of the 8-bit
  // codec: clamp(floor((r - lut_lo) * lut_inv_w), 0, TURBO_LUT_BUCKETS - 1);
  // lut_ok = 0 when the buckets would be wider than the smallest gap
  // between two thresholds (then the kernels search the thresholds).
  float lut_lo, lut_inv_w;
  int lut_ok;
};
constexpr int TURBO_LUT_BUCKETS = 1024;

// Lloyd-Max levels of the standard normal with 2^bits levels (host, f64).
void lloyd_max_normal(int bits, double* levels);
// The f32 table of an (n, bits) codec.
void turbo_table(int n, int bits, TurboTable* t);

}  // namespace hq
