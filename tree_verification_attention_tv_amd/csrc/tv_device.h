// Device helpers shared by the kernels (host-only sources do not include this).
#pragma once

#include "tv_internal.h"

namespace tv {

// sets error bits in the caller's device error word (when one is given)
__device__ __forceinline__ void raise_err(int32_t* dev_err, int bits) {
  if (dev_err) atomicOr(dev_err, bits);
}

}  // namespace tv
