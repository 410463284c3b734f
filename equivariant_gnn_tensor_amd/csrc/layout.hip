// Feature layouts at the boundary: mul_ir <-> ir_mul.
//
// The kernels keep every irrep block of a feature row as [2l+1][C] with the channels of
// one component adjacent (ir_mul); the common default elsewhere is [C][2l+1] (mul_ir).
// Converting is a transpose of each block, row by row (Sobek paper, Sec. 4, the
// implementation paragraph: the wrapper transposes at the boundary, or callers keep
// ir_mul across layers).  Pure data movement, so it is HBM bound.  A workgroup stages a
// strip of whole rows in LDS with 16-byte coalesced loads, then each thread maps four
// adjacent output columns to their source columns once and writes them as one 16-byte
// store per row of the strip; the permutation happens in LDS, not in the gathers.  Rows
// wider than the LDS budget fall back to a direct kernel that gathers from global memory.
#include <algorithm>
#include <cstdint>
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

constexpr int kLdsFloats = 8192;   // 32 KB of LDS per workgroup: several workgroups per CU

// Rows [r0, r0 + R) staged in LDS; VEC: width % 4 == 0 and 16-byte aligned pointers.
template <bool VEC>
__global__ __launch_bounds__(kLayoutThreads) void layout_lds_kernel(const float* __restrict__ in,
                                                                   float* __restrict__ out, int64_t n_rows,
                                                                   const LayoutBlocks t, int to_ir_mul, int R) {
  __shared__ float lds[kLdsFloats];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * R;
  const int nr = static_cast<int>(std::min<int64_t>(R, n_rows - r0));
  const int32_t dim = t.dim;
  const int total = nr * dim;
  const int64_t base = r0 * dim;
  if (VEC) {
    const float4* src4 = reinterpret_cast<const float4*>(in + base);
    for (int i = threadIdx.x; i < total / 4; i += kLayoutThreads) {
      const float4 v = src4[i];
      lds[4 * i] = v.x;
      lds[4 * i + 1] = v.y;
      lds[4 * i + 2] = v.z;
      lds[4 * i + 3] = v.w;
    }
  } else {
    for (int i = threadIdx.x; i < total; i += kLayoutThreads) lds[i] = in[base + i];
  }
  __syncthreads();
  if (VEC) {
    for (int32_t c = 4 * threadIdx.x; c < dim; c += 4 * kLayoutThreads) {
      const int32_t s0 = source_col(c, t, to_ir_mul), s1 = source_col(c + 1, t, to_ir_mul);
      const int32_t s2 = source_col(c + 2, t, to_ir_mul), s3 = source_col(c + 3, t, to_ir_mul);
      for (int r = 0; r < nr; ++r) {
        const float* row = lds + r * dim;
        *reinterpret_cast<float4*>(out + base + static_cast<int64_t>(r) * dim + c) =
            make_float4(row[s0], row[s1], row[s2], row[s3]);
      }
    }
  } else {
    for (int32_t c = threadIdx.x; c < dim; c += kLayoutThreads) {
      const int32_t sc = source_col(c, t, to_ir_mul);
      for (int r = 0; r < nr; ++r) out[base + static_cast<int64_t>(r) * dim + c] = lds[r * dim + sc];
    }
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
  const int to_ir_mul = direction == ETPC_TO_IR_MUL ? 1 : 0;
  ::etpc::ProfScope ps(ETPC_KIND_PREP, s);
  if (off <= kLdsFloats) {
    const int R = std::min(64, kLdsFloats / off);
    const int64_t groups = (static_cast<int64_t>(n_rows) + R - 1) / R;
    const bool vec = off % 4 == 0 && (reinterpret_cast<uintptr_t>(in) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    if (vec)
      hipLaunchKernelGGL(layout_lds_kernel<true>, dim3(static_cast<unsigned>(groups)), dim3(kLayoutThreads), 0, s, in,
                         out, static_cast<int64_t>(n_rows), t, to_ir_mul, R);
    else
      hipLaunchKernelGGL(layout_lds_kernel<false>, dim3(static_cast<unsigned>(groups)), dim3(kLayoutThreads), 0, s,
                         in, out, static_cast<int64_t>(n_rows), t, to_ir_mul, R);
  } else {
    const int64_t groups = (static_cast<int64_t>(n_rows) + kRowsPerGroup - 1) / kRowsPerGroup;
    hipLaunchKernelGGL(layout_kernel, dim3(static_cast<unsigned>(groups)), dim3(kLayoutThreads), 0, s, in, out,
                       static_cast<int64_t>(n_rows), t, to_ir_mul);
  }
  ETPC_HIP(hipGetLastError());
  return ETPC_OK;
}

}  // namespace etpc
