// lla_dispatch.hpp — kernel tables shared by the C-ABI host code and the instantiation units.
#pragma once

namespace lla {

struct KernelSet {
  const void* fwd[2];        // lla_fwd_kernel<T, C, DK, DV, NB, false> for NB = 1, 2 resident chunks
  const void* fwd_varlen[2]; // lla_fwd_kernel<T, C, DK, DV, NB, true>: variable-length batches
};

// dtype 0 = bf16, 1 = f32; C, DK, DV in {16, 32, 64, 128}; nullptr otherwise.
const KernelSet* kernel_set(int dtype, int C, int DK, int DV);

// per (dtype, C) tables, one instantiation unit each
const KernelSet* kernels_bf16_c16(int DK, int DV);
const KernelSet* kernels_bf16_c32(int DK, int DV);
const KernelSet* kernels_bf16_c64(int DK, int DV);
const KernelSet* kernels_bf16_c128(int DK, int DV);
const KernelSet* kernels_f32_c16(int DK, int DV);
const KernelSet* kernels_f32_c32(int DK, int DV);
const KernelSet* kernels_f32_c64(int DK, int DV);
const KernelSet* kernels_f32_c128(int DK, int DV);

inline int dim_index(int x) { return x == 16 ? 0 : x == 32 ? 1 : x == 64 ? 2 : x == 128 ? 3 : -1; }

}  // namespace lla
