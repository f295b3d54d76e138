// lla_inst.hpp — builds one (dtype, chunk) table of kernel instantiations.
#pragma once
#include <type_traits>

#include "lla_dispatch.hpp"
#include "lla_kernels.hpp"

namespace lla {

// The shared-memory-aliasing output kernel exists only where the plain one cannot fit:
// bf16, C = 128, dk = dv = 128.
template <typename TY, int C, int DK, int DV>
const void* alias_kernel() {
  if constexpr (std::is_same<TY, bf16>::value && C == 128 && DK == 128 && DV == 128)
    return reinterpret_cast<const void*>(&lla_query_kernel<TY, C, DK, DV, true>);
  else
    return nullptr;
}

template <typename TY, int C, int DK, int DV>
KernelSet make_set() {
  return KernelSet{reinterpret_cast<const void*>(&lla_sweep_state_kernel<TY, C, DK, DV>),
                   reinterpret_cast<const void*>(&lla_fenwick_kernel<TY, DK, DV>),
                   reinterpret_cast<const void*>(&lla_query_kernel<TY, C, DK, DV, false>),
                   alias_kernel<TY, C, DK, DV>()};
}

template <typename TY, int C, int DK>
struct Row {
  static void fill(KernelSet (&r)[4]) {
    r[0] = make_set<TY, C, DK, 16>();
    r[1] = make_set<TY, C, DK, 32>();
    r[2] = make_set<TY, C, DK, 64>();
    r[3] = make_set<TY, C, DK, 128>();
  }
};

template <typename TY, int C>
const KernelSet* table_lookup(int DK, int DV) {
  static const struct Table {
    KernelSet t[4][4];
    Table() {
      Row<TY, C, 16>::fill(t[0]);
      Row<TY, C, 32>::fill(t[1]);
      Row<TY, C, 64>::fill(t[2]);
      Row<TY, C, 128>::fill(t[3]);
    }
  } table;
  const int di = dim_index(DK), vi = dim_index(DV);
  if (di < 0 || vi < 0) return nullptr;
  return &table.t[di][vi];
}

}  // namespace lla
