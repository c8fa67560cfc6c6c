// Placement of a model's routed experts between HBM and pinned host memory.
//
// The hipfire expert-offload explainer, section "放置算法：auto 自动放置…",
// gives the rules: the fixed (non-expert) weights go first; then, by
// default, routed experts fill the device budget layer by layer ("fit-
// capacity placement") and the remaining layers stay in pinned host memory;
// a hot-set ranking by decode frequency lets the device hold the most often
// selected experts instead of whole layers; and a configuration that does
// not fit is refused at load time, naming what is short and by how many
// bytes.  The Strata user report, sections "1. Strata 是什么" and "5. 实测速度",
// caches the most routed experts on the device and reports the cache's hit
// rate.  Both modes are implemented here on the host; the device side only
// follows the resulting per-expert pointers.
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "placement.h"

namespace hq {

int place_experts(int mode, int64_t layers, int64_t E, const uint64_t* heat,
                  uint64_t expert_bytes, uint64_t fixed_bytes, uint64_t budget_bytes,
                  uint8_t* resident, uint64_t* placed_bytes, uint64_t* short_bytes) {
  const int64_t n = layers * E;
  std::fill(resident, resident + n, (uint8_t)0);
  *placed_bytes = 0;
  *short_bytes = 0;
  if (fixed_bytes > budget_bytes) {
    *short_bytes = fixed_bytes - budget_bytes;
    return 1;   // does not fit: the caller refuses with the shortfall
  }
  uint64_t left = budget_bytes - fixed_bytes;
  if (mode == 0) {
    // whole layers in order while a layer's experts fit
    const uint64_t layer_bytes = expert_bytes * (uint64_t)E;
    for (int64_t l = 0; l < layers && layer_bytes <= left; ++l) {
      std::fill(resident + l * E, resident + (l + 1) * E, (uint8_t)1);
      left -= layer_bytes;
      *placed_bytes += layer_bytes;
    }
    return 0;
  }
  // single experts, hottest first; equal heat goes to the lower (layer,
  // expert) index, so the placement is a pure function of the counts
  std::vector<int64_t> order(n);
  std::iota(order.begin(), order.end(), (int64_t)0);
  std::stable_sort(order.begin(), order.end(),
                   [heat](int64_t a, int64_t b) { return heat[a] > heat[b]; });
  for (int64_t i = 0; i < n && expert_bytes <= left; ++i) {
    resident[order[i]] = 1;
    left -= expert_bytes;
    *placed_bytes += expert_bytes;
  }
  return 0;
}

}  // namespace hq
