// lla_host.hpp — host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <stdlib.h>

namespace lla {

// Stream-ordered workspace allocation of the entry points that take their workspace themselves.
// With LLA_TEST_FAIL_ALLOC=1 in the environment it fails before touching the device, so that the
// LLA_ERR_NO_MEMORY path can be exercised on a machine without a GPU.
inline hipError_t workspace_alloc(void** p, size_t bytes, hipStream_t stream) {
  const char* f = getenv("LLA_TEST_FAIL_ALLOC");
  if (f && f[0] == '1' && f[1] == '\0') return hipErrorOutOfMemory;
  return hipMallocAsync(p, bytes, stream);
}

constexpr int kLdsPerCU = 160 * 1024;      // gfx950 shared memory per compute unit (and workgroup)

}  // namespace lla
