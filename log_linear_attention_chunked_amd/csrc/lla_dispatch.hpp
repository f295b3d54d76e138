// lla_dispatch.hpp — kernel tables shared by the C-ABI host code and the instantiation units.
#pragma once

namespace lla {

struct KernelSet {
  const void* state;         // lla_sweep_state_kernel<T, C, DK>
  const void* fenwick;       // lla_fenwick_kernel<T, DK>
  const void* query;         // lla_query_kernel<T, C, DK, false>
  const void* query_alias;   // lla_query_kernel<T, C, DK, true>, or nullptr
};

// C in {16, 32, 64, 128}, DK in {16, 32, 64, 128}; nullptr otherwise.
const KernelSet* kernels_bf16(int C, int DK);
const KernelSet* kernels_f32(int C, int DK);

}  // namespace lla
