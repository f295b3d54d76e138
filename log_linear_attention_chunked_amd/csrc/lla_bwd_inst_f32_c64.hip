// Backward-pass kernel instantiations: f32 q/k/v/do and gradients, chunk size 64, all head dims.
#include "lla_bwd.hpp"

namespace lla {
namespace bwd {
const BwdKernels* bwd_kernels_f32_c64(int DK, int DV) { return bwd_table<float, 64>(DK, DV); }
}  // namespace bwd
}  // namespace lla
