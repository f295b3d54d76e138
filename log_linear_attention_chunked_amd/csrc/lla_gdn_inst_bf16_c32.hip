// Log-linear Gated DeltaNet kernels for bf16 inputs, chunk 32: one instantiation unit.
#include "lla_gdn.hpp"

const lla::gdn::GdnKernels* lla::gdn::kernels_bf16_c32(int DK, int DV) {
  static const GdnTable<lla::gdn::bf16, 32> table;
  return table.get(DK, DV);
}
