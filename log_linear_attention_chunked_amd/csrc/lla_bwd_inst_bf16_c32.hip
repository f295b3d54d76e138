// Backward-pass kernel instantiations: bf16 q/k/v/do and gradients, chunk size 32, all head dims.
#include "lla_bwd.hpp"

namespace lla {
namespace bwd {
const BwdKernels* bwd_kernels_bf16_c32(int DK, int DV) { return bwd_table<bf16, 32>(DK, DV); }
}  // namespace bwd
}  // namespace lla
