// Wavefront-level helpers for gfx950 (wave64): DPP row reductions.
#pragma once

#include <hip/hip_runtime.h>

namespace etpc {

template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Three row sums at once: every lane of each 16-lane row receives the sum over that row
// of each value (row_ror rotations by 8, 4, 2, 1).  The three chains are interleaved, so
// each DPP step reads a value written two instructions earlier, which covers the DPP
// read-after-write wait states without s_nop.
__device__ inline void row_sum16x3(float& a, float& b, float& c) {
  a += dpp_f<0x128>(a);
  b += dpp_f<0x128>(b);
  c += dpp_f<0x128>(c);
  a += dpp_f<0x124>(a);
  b += dpp_f<0x124>(b);
  c += dpp_f<0x124>(c);
  a += dpp_f<0x122>(a);
  b += dpp_f<0x122>(b);
  c += dpp_f<0x122>(c);
  a += dpp_f<0x121>(a);
  b += dpp_f<0x121>(b);
  c += dpp_f<0x121>(c);
}

}  // namespace etpc
