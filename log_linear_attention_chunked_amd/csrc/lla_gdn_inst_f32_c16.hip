// Log-linear Gated DeltaNet kernels for f32 inputs, chunk 16: one instantiation unit.
#include "lla_gdn.hpp"

const lla::gdn::GdnKernels* lla::gdn::kernels_f32_c16(int DK, int DV) {
  static const GdnTable<float, 16> table;
  return table.get(DK, DV);
}
