// Wavefront-level helpers for gfx950 (wave64): DPP row reductions.
#pragma once

#include <hip/hip_runtime.h>

namespace etpc {

template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Every lane of each 16-lane row receives the sum over that row (row_ror rotations).
__device__ inline float row_sum16(float v) {
  v += dpp_f<0x128>(v);  // row_ror:8
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x122>(v);  // row_ror:2
  v += dpp_f<0x121>(v);  // row_ror:1
  return v;
}

}  // namespace etpc
