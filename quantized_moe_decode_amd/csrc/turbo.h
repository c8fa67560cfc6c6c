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
  // Bucket of a value r for the encoder's nearest-level search:
  // clamp(fma(r, lut_a, lut_b), 0, turbo_lut_buckets(bits) - 1) truncated
  // (a monotone map).  lut_ok = 0 when the buckets would not be narrower
  // than half the smallest gap between two thresholds (then the encoder
  // searches the thresholds).
  float lut_a, lut_b;
  int lut_ok;
};
// Buckets of the encoder's table: enough for half the smallest threshold
// gap of the Lloyd-Max levels (2 range / gap is 4, 14, 37 and 1075 for 2,
// 3, 4 and 8 bits), and no more, so that the table's byte reads at
// data-dependent entries stay within few LDS words.
constexpr int turbo_lut_buckets(int bits) { return bits <= 4 ? 128 : 2048; }

// Lloyd-Max levels of the standard normal with 2^bits levels (host, f64).
void lloyd_max_normal(int bits, double* levels);
// The f32 table of an (n, bits) codec.
void turbo_table(int n, int bits, TurboTable* t);

}  // namespace hq
