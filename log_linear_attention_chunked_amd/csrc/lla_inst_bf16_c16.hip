// Kernel instantiations: bf16 q/k/v/out, chunk size 16, all head dims.
#include "lla_inst.hpp"

namespace lla {
const KernelSet* kernels_bf16_c16(int DK, int DV) { return table_lookup<bf16, 16>(DK, DV); }
}  // namespace lla
