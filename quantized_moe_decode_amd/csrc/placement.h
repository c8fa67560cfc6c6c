// Expert placement between HBM and pinned host memory (host only).
#pragma once
#include <stdint.h>

namespace hq {

// mode 0: whole layers in order while the budget lasts; mode 1: single
// experts by heat (hottest first, ties to the lower index).  resident[l*E+e]
// receives 1 for experts placed in HBM.  Returns 1 (and *short_bytes) when
// the fixed bytes alone exceed the budget, else 0.
int place_experts(int mode, int64_t layers, int64_t E, const uint64_t* heat,
                  uint64_t expert_bytes, uint64_t fixed_bytes, uint64_t budget_bytes,
                  uint8_t* resident, uint64_t* placed_bytes, uint64_t* short_bytes);

}  // namespace hq
