// Kernel instantiations: f32 q/k/v/out, chunk size 32, all head dims.
#include "lla_inst.hpp"

namespace lla {
const KernelSet* kernels_f32_c32(int DK, int DV) { return table_lookup<float, 32>(DK, DV); }
}  // namespace lla
