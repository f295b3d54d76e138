// Kernel instantiations: bf16 q/k/v/out, chunk size 64, all head dims.
#include "lla_inst.hpp"

namespace lla {
const KernelSet* kernels_bf16_c64(int DK, int DV) { return table_lookup<bf16, 64>(DK, DV); }
}  // namespace lla
