// Planner: irreps spec -> paths, coupling tensors, offsets (host only).
#pragma once

#include <vector>

#include "common.hpp"

namespace etpc {

struct PathInfo {
  int32_t in_block, l_sh, out_block;
  int32_t l_in, l_out;
  int32_t c_in, c_out;
  int64_t w_off, w_numel;
  int32_t fan_in;
  int32_t pos_in_group;   // index among the paths of its output block (plan order)
  int32_t pos_in_block;   // index among the paths of its input block (plan order)
  double cg[7 * 7 * 7];   // dense [2l_in+1][2l_sh+1][2l_out+1]
  CGTable cgf;            // float copy, [NI][7][NO]
};

}  // namespace etpc

struct etpc_plan_s {
  std::vector<etpc_irrep> in, out;
  std::vector<int64_t> xoff, zoff;
  int32_t lmax_sh = 0, mode = 0, radial = 0, n_basis = 0, poly_p = 0;
  float r_lo = 0.f, r_hi = 0.f;
  float box[3] = {0.f, 0.f, 0.f};
  bool periodic = false;
  int32_t gemm_precision = 0;   // etpc_gemm_precision of the channel GEMMs
  int32_t lanes = 2;            // concurrent launch lanes of a pass (1 = serialized)
  int64_t x_dim = 0, z_dim = 0, w_numel = 0;
  std::vector<etpc::PathInfo> paths;
  // paths grouped by output block / input block (indices into `paths`, plan order)
  std::vector<std::vector<int>> by_out, by_in;
  etpc::GeomParams geom() const;
};

namespace etpc {
// Real-basis coupling tensor of (l1, l2, l3) in float64 via Racah's formula; out is
// [2l1+1][2l2+1][2l3+1].  Returns false if the triangle rule fails.
bool real_cg_racah(int l1, int l2, int l3, double* out);
}  // namespace etpc
