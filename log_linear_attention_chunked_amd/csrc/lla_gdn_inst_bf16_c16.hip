// Log-linear Gated DeltaNet kernels for bf16 inputs, chunk 16: one instantiation unit.
#include "lla_gdn.hpp"

const lla::gdn::GdnKernels* lla::gdn::kernels_bf16_c16(int DK, int DV) {
  static const GdnTable<lla::gdn::bf16, 16> table;
  return table.get(DK, DV);
}
