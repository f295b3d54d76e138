// Instantiations of the forward-pass kernels with f32 q, k, v, out.
#include "lla_dispatch.hpp"
#include "lla_kernels.hpp"

namespace lla {

#define LLA_SET(C, DK, ALIAS)                                                        \
  KernelSet {                                                                        \
    reinterpret_cast<const void*>(&lla_sweep_state_kernel<float, C, DK>),             \
    reinterpret_cast<const void*>(&lla_fenwick_kernel<float, DK>),                    \
    reinterpret_cast<const void*>(&lla_query_kernel<float, C, DK, false>),            \
    ALIAS ? reinterpret_cast<const void*>(&lla_query_kernel<float, C, DK, ALIAS>) : nullptr \
  }

const KernelSet* kernels_f32(int C, int DK) {
  static const KernelSet table[4][4] = {
    {LLA_SET(16, 16, false), LLA_SET(16, 32, false), LLA_SET(16, 64, false), LLA_SET(16, 128, false)},
    {LLA_SET(32, 16, false), LLA_SET(32, 32, false), LLA_SET(32, 64, false), LLA_SET(32, 128, false)},
    {LLA_SET(64, 16, false), LLA_SET(64, 32, false), LLA_SET(64, 64, true), LLA_SET(64, 128, true)},
    {LLA_SET(128, 16, false), LLA_SET(128, 32, false), LLA_SET(128, 64, true), LLA_SET(128, 128, true)},
  };
  auto idx = [](int x) { return x == 16 ? 0 : x == 32 ? 1 : x == 64 ? 2 : x == 128 ? 3 : -1; };
  const int ci = idx(C), di = idx(DK);
  if (ci < 0 || di < 0) return nullptr;
  return &table[ci][di];
}

}  // namespace lla
