// noalloc.h -- the static device scratch behind pa_decode_step_noalloc
// (internal).
#pragma once

#include <cstddef>

#include <hip/hip_runtime.h>

namespace pa {

// Size of the file-scope device array in noalloc.hip (per device).
inline constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;

// The current device's address of that array, looked up on the first call
// on each device (hipGetSymbolAddress with the device current) and kept.
hipError_t noalloc_scratch(void** out);

}  // namespace pa
