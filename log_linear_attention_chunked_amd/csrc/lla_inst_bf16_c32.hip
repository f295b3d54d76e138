// Kernel instantiations: bf16 q/k/v/out, chunk size 32, all head dims.
#include "lla_inst.hpp"

namespace lla {
const KernelSet* kernels_bf16_c32(int DK, int DV) { return table_lookup<bf16, 32>(DK, DV); }
}  // namespace lla
