// Kernel instantiations: f32 q/k/v/out, chunk size 128, all head dims.
#include "lla_inst.hpp"

namespace lla {
const KernelSet* kernels_f32_c128(int DK, int DV) { return table_lookup<float, 128>(DK, DV); }
}  // namespace lla
