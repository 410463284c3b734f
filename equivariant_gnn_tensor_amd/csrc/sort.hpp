// Integer building blocks of the graph preparation steps (internal, defined in csr.hip):
// a stable least-significant-digit radix sort of (key, value) int32 pairs with 8-bit
// digits, an exclusive scan, and small copy and lower-bound launches.  All of them are
// deterministic and bit-exact (LDS atomics only count).
#pragma once

#include "common.hpp"

namespace etpc {

// k0/v0 hold the input; the sorted result lands in (k0, v0) after the call (the
// pointers are swapped per pass).  hist and aux need sort_scratch_ints(n) ints together,
// hist first (256 per tile of items), aux right after it.
struct SortBufs {
  int32_t *k0, *v0, *k1, *v1, *hist, *aux;
};

// Buffers for sorting n items: hist and aux are carved from `scratch`
// (sort_scratch_ints(n) ints).
SortBufs make_sort_bufs(int32_t* k0, int32_t* v0, int32_t* k1, int32_t* v1, int32_t* scratch, int64_t n);

int grid_for(int64_t n, int block);
size_t scan_aux_ints(int64_t n);
size_t sort_scratch_ints(int64_t n);
// Number of 8-bit digit passes for keys in [0, n_keys).
int radix_passes(int32_t n_keys);
hipError_t radix_sort(SortBufs& b, int64_t n, int passes, hipStream_t s);
// In-place exclusive scan of n ints; aux holds scan_aux_ints(n) ints.
hipError_t exclusive_scan(int32_t* data, int64_t n, int32_t* aux, hipStream_t s);
hipError_t launch_copy(const int32_t* a, int32_t* b, int64_t n, hipStream_t s);
// rowptr[v] = first index whose key is >= v, v = 0..n_rows (keys sorted ascending)
hipError_t launch_lower_bound(const int32_t* keys, int64_t n, int32_t* rowptr, int32_t n_rows, hipStream_t s);

}  // namespace etpc
