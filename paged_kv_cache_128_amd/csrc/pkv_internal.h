// Internal declarations shared by the host sources of libpkv (not installed).
#pragma once
#include <stdint.h>
#include <stddef.h>
#include "pkv.h"

namespace pkv {

inline int elem_bytes(int dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

// Validate a cache layout; returns PKV_OK or PKV_ERR_INVALID.
int check_layout(const pkv_cache_layout* l);

// One decode step's host metadata, carried into a launch as kernel
// arguments: per row the new token's slot and the row's length after the
// append.
constexpr int kStepRows = 256;
struct StepMeta {
  int64_t slots[kStepRows];
  int32_t lens[kStepRows];
};

}  // namespace pkv
