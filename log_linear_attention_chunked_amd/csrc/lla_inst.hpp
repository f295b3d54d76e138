// lla_inst.hpp — builds one (dtype, chunk) table of kernel instantiations.
#pragma once

#include "lla_dispatch.hpp"
#include "lla_kernels.hpp"

namespace lla {

template <typename TY, int C, int DK, int DV>
KernelSet make_set() {
  return KernelSet{{reinterpret_cast<const void*>(&lla_fwd_kernel<TY, C, DK, DV, 1, false>),
                    reinterpret_cast<const void*>(&lla_fwd_kernel<TY, C, DK, DV, 2, false>)},
                   {reinterpret_cast<const void*>(&lla_fwd_kernel<TY, C, DK, DV, 1, true>),
                    reinterpret_cast<const void*>(&lla_fwd_kernel<TY, C, DK, DV, 2, true>)}};
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
