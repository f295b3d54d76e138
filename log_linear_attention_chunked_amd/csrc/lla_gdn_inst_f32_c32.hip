// Log-linear Gated DeltaNet kernels for f32 inputs, chunk 32: one instantiation unit.
#include "lla_gdn.hpp"

const lla::gdn::GdnKernels* lla::gdn::kernels_f32_c32(int DK, int DV) {
  static const GdnTable<float, 32> table;
  return table.get(DK, DV);
}
