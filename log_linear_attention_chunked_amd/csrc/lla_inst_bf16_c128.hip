// Kernel instantiations: bf16 q/k/v/out, chunk size 128, all head dims.
#include "lla_inst.hpp"

namespace lla {
const KernelSet* kernels_bf16_c128(int DK, int DV) { return table_lookup<bf16, 128>(DK, DV); }
}  // namespace lla
