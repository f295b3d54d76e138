// Log-linear Gated DeltaNet kernels for f32 inputs, chunk 64: one instantiation unit.
#include "lla_gdn.hpp"

const lla::gdn::GdnKernels* lla::gdn::kernels_f32_c64(int DK, int DV) {
  static const GdnTable<float, 64> table;
  return table.get(DK, DV);
}
