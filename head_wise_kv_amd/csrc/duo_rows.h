// Where a retrieval head's row lives, for the two layouts of the arena
// (contiguous rows per head, or pages named by a per-row page table).  Shared
// by the HIP kernels; the host never computes device row addresses itself.
#pragma once

#include "duo_internal.h"

namespace duo {

// Row number, within the layer's retrieval K (or V) array, of position p of
// compact retrieval head r of batch row b.  Contiguous: row p of the head's
// cap_ret rows.  Paged: row p mod page rows of the head's part of the page
// that the table names for p's page of batch row b.
__device__ __forceinline__ int64_t ret_row(const LayerPtrs& lp, int n_ret, int64_t cap_ret, int64_t b, int r,
                                           int64_t p) {
  if (lp.table) {
    const int64_t page = lp.table[b * lp.max_pages + (p >> lp.page_shift)];
    return ((page * n_ret + r) << lp.page_shift) + (p & ((int64_t{1} << lp.page_shift) - 1));
  }
  return (b * n_ret + r) * cap_ret + p;
}

// Row, counted from a paged head's rows in page 0, of position p, for a
// wavefront-uniform p: the table entry is read through the scalar cache
// (valid because no kernel that reads a table this way writes it), so the
// read adds nothing to the vector-memory counter.
__device__ __forceinline__ int64_t paged_row(const int32_t* row_table, int shift, int64_t page_stride, int64_t p) {
  const int32_t page = *(const __attribute__((address_space(4))) int32_t*)(row_table + (p >> shift));
  return (int64_t)page * page_stride + (p & ((int64_t{1} << shift) - 1));
}

// Whether batch row b, holding `cnt` tokens, has room for n more: within
// T_cap and, for paged retrieval rows, on pages the row's table names (a
// row's table names the pages of a prefix of its positions; the entries past
// them hold -1).
__device__ __forceinline__ bool room_for(const LayerPtrs& lp, int64_t b, int64_t cnt, int64_t n) {
  if (cnt + n > lp.cap) return false;
  if (lp.table && n > 0) return lp.table[b * lp.max_pages + ((cnt + n - 1) >> lp.page_shift)] >= 0;
  return true;
}

}  // namespace duo
