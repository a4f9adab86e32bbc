// Budget of one query head's critical set T_t.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico",
// "Variantes de Implementacao": FASA composes with allocating the budget
// across layers.  A call may give each query head its own budget (a device
// array); without one every head takes the call's budget.
#pragma once

#include "device_common.hpp"

namespace fasa {

// Budget of query head h: head_budget[h] when a per-head array is given, else
// the call's budget.  A per-head value outside [0, budget] is clamped into it
// and raises flag 8 (if report).
__device__ __forceinline__ int row_budget(const int32_t* head_budget, int h, int budget,
                                          uint32_t* err, bool report) {
  if (head_budget == nullptr) return budget;
  const int v = head_budget[h];
  if (v < 0 || v > budget) {
    if (report) raise_flag(err, 8u);
    return v < 0 ? 0 : budget;
  }
  return v;
}

}  // namespace fasa
