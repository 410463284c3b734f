// Feature layouts at the boundary: mul_ir <-> ir_mul.
//
// The kernels keep every irrep block of a feature row as [2l+1][C] with the channels of
// one component adjacent (ir_mul); the common default elsewhere is [C][2l+1] (mul_ir).
// Converting is a transpose of each block, row by row (Sobek paper, Sec. 4, the
// implementation paragraph: the wrapper transposes at the boundary, or callers keep
// ir_mul across layers).  Pure data movement, so it is HBM bound: each workgroup owns a
// strip of rows; a thread maps each of its output columns to the source column once and
// then streams that column through the strip, so stores are coalesced and the gathered
// loads of one row stay inside the cache lines the row occupies.
#include <algorithm>
#include <vector>

#include "kernels.hpp"
#include "profile.hpp"

namespace etpc {
namespace {

constexpr int kLayoutThreads = 256;
constexpr int kMaxLayoutBlocks = 64;
constexpr int kRowsPerGroup = 16;

// Consecutive blocks that need no transpose (l = 0 or C = 1) are merged into one copy
// block (d = 1).
struct LayoutBlocks {
  int32_t n;
  int32_t dim;
  int32_t off[kMaxLayoutBlocks + 1];
  int32_t mul[kMaxLayoutBlocks];
  int32_t d[kMaxLayoutBlocks];
};

// Source column of output column c.  to_ir_mul: output (m, u) at m C + u reads
// mul_ir u d + m; otherwise output (u, m) at u d + m reads ir_mul m C + u.
__device__ inline int32_t source_col(int32_t c, const LayoutBlocks& t, int to_ir_mul) {
  int b = 0;
  while (b + 1 < t.n && t.off[b + 1] <= c) ++b;
  const int32_t loc = c - t.off[b];
  const int32_t C = t.mul[b], d = t.d[b];
  if (d == 1) return c;
  if (to_ir_mul) {
    const int32_t m = loc / C, u = loc - m * C;
    return t.off[b] + u * d + m;
  }
  const int32_t u = loc / d, m = loc - u * d;
  return t.off[b] + m * C + u;
}

__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                               int64_t n_rows, const LayoutBlocks t, int to_ir_mul) {
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerGroup;
  const int64_t r1 = std::min<int64_t>(r0 + kRowsPerGroup, n_rows);
  for (int32_t c = threadIdx.x; c < t.dim; c += kLayoutThreads) {
    const int32_t sc = source_col(c, t, to_ir_mul);
    for (int64_t r = r0; r < r1; ++r) out[r * t.dim + c] = in[r * t.dim + sc];
  }
}

}  // namespace

etpc_status layout_convert_impl(const std::vector<etpc_irrep>& irreps, int direction, int32_t n_rows,
                                const float* in, float* out, hipStream_t s) {
  LayoutBlocks t{};
  int32_t off = 0;
  for (const etpc_irrep& ir : irreps) {
    const int32_t d = 2 * ir.l + 1;
    const bool copy = ir.l == 0 || ir.mul == 1;
    if (copy && t.n > 0 && t.d[t.n - 1] == 1) {
      off += ir.mul * d;   // extend the open copy block
      continue;
    }
    if (t.n == kMaxLayoutBlocks) ETPC_FAIL(ETPC_ERR_UNSUPPORTED, "layout conversion supports at most 64 blocks");
    t.off[t.n] = off;
    t.mul[t.n] = copy ? ir.mul * d : ir.mul;
    t.d[t.n] = copy ? 1 : d;
    ++t.n;
    off += ir.mul * d;
  }
  t.off[t.n] = off;
  t.dim = off;
  if (n_rows == 0 || off == 0) return ETPC_OK;
  const int64_t groups = (static_cast<int64_t>(n_rows) + kRowsPerGroup - 1) / kRowsPerGroup;
  ::etpc::ProfScope ps(ETPC_KIND_PREP, s);
  hipLaunchKernelGGL(layout_kernel, dim3(static_cast<unsigned>(groups)), dim3(kLayoutThreads), 0, s, in, out,
                     static_cast<int64_t>(n_rows), t, direction == ETPC_TO_IR_MUL ? 1 : 0);
  ETPC_HIP(hipGetLastError());
  return ETPC_OK;
}

}  // namespace etpc
