// Small memory-bound helpers: fill, weight re-layout, fixed-order reductions.
#include "kernels.hpp"

namespace etpc {
namespace {

__global__ void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

// one path per blockIdx.y: wcat[u][col0 + q*cout + w], wt[(col0 + q*cout + w)][u] from W[q][u][w]
__global__ void wprep_kernel(const WPrepArgs a) {
  const int t = blockIdx.y;
  const int cout = a.cout[t];
  const int64_t per_path = static_cast<int64_t>(a.nb) * a.c_in * cout;
  const float* w = a.w + a.path_off[t];
  for (int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; r < per_path;
       r += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int q = static_cast<int>(r / (static_cast<int64_t>(a.c_in) * cout));
    const int64_t rr = r - static_cast<int64_t>(q) * a.c_in * cout;
    const int u = static_cast<int>(rr / cout);
    const int wch = static_cast<int>(rr - static_cast<int64_t>(u) * cout);
    const float v = w[r];
    const int64_t col = a.col0[t] + static_cast<int64_t>(q) * cout + wch;
    if (a.wcat) a.wcat[static_cast<int64_t>(u) * a.ncols + col] = v;
    if (a.wt) a.wt[col * a.c_in + u] = v;
  }
}

struct ReduceWArgs {
  const float* part;
  int32_t splits, split_step, rows, ncols, nb;
  int32_t accumulate;
  float* out;
  int64_t path_off[kMaxPaths];
  int32_t col0[kMaxPaths];
  int32_t cout[kMaxPaths];
};

// Early stage for many partial copies: of the `splits` copies held at copies 0, step,
// 2 step, ..., group g = blockIdx.y sums copies [g*seg, (g+1)*seg) of each element in order
// and stores the sum over copy g*seg*step (only this thread reads or writes that element's
// copies in the group, so the update is in place).
__global__ void segment_sum_kernel(float* __restrict__ part, int splits, int seg, int64_t stride, int step) {
  const int64_t c = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (c >= stride) return;
  const int z0 = blockIdx.y * seg;
  const int z1 = min(splits, z0 + seg);
  const int64_t zs = static_cast<int64_t>(step) * stride;
  float* p = part + static_cast<int64_t>(z0) * zs + c;
  float s = 0.f;
  for (int z = z0; z < z1; ++z) s += p[static_cast<int64_t>(z - z0) * zs];
  *p = s;
}

// one path per blockIdx.y; element r of the path block = (q, u, w) in W order
__global__ void reduce_wbar_kernel(const ReduceWArgs a) {
  const int t = blockIdx.y;
  const int cout = a.cout[t];
  const int64_t per_path = static_cast<int64_t>(a.nb) * a.rows * cout;
  const int64_t split_stride = static_cast<int64_t>(a.rows) * a.ncols;
  for (int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; r < per_path;
       r += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int q = static_cast<int>(r / (static_cast<int64_t>(a.rows) * cout));
    const int64_t rr = r - static_cast<int64_t>(q) * a.rows * cout;
    const int u = static_cast<int>(rr / cout);
    const int w = static_cast<int>(rr - static_cast<int64_t>(u) * cout);
    const int64_t src = static_cast<int64_t>(u) * a.ncols + a.col0[t] + static_cast<int64_t>(q) * cout + w;
    float s = 0.f;
    for (int z = 0; z < a.splits; ++z) s += a.part[static_cast<int64_t>(z) * a.split_step * split_stride + src];
    float* o = a.out + a.path_off[t] + r;
    *o = a.accumulate ? (*o + s) : s;
  }
}

// one wavefront per node: lanes stride over the node's sender and receiver slots; the lane
// partials are combined by a fixed reduction tree (deterministic).  rbar holds `copies`
// per-lane copies of the edge adjoint (stride floats apart), summed in copy order.
__global__ __launch_bounds__(256) void pos_bar_kernel(const int32_t* __restrict__ rowptr,
                                                     const int32_t* __restrict__ s_rowptr,
                                                     const int32_t* __restrict__ s_slot,
                                                     const float* __restrict__ rbar, int copies, int64_t stride,
                                                     float* __restrict__ pos_bar, int n) {
  const int v = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (v >= n) return;
  float sx = 0.f, sy = 0.f, sz = 0.f;
  for (int k = s_rowptr[v] + lane; k < s_rowptr[v + 1]; k += 64) {
    const float* r = rbar + 3 * static_cast<int64_t>(s_slot[k]);
    float ex = 0.f, ey = 0.f, ez = 0.f;
    for (int c = 0; c < copies; ++c) {
      ex += r[c * stride + 0];
      ey += r[c * stride + 1];
      ez += r[c * stride + 2];
    }
    sx += ex;
    sy += ey;
    sz += ez;
  }
  for (int64_t e = rowptr[v] + lane; e < rowptr[v + 1]; e += 64) {
    const float* r = rbar + 3 * e;
    float ex = 0.f, ey = 0.f, ez = 0.f;
    for (int c = 0; c < copies; ++c) {
      ex += r[c * stride + 0];
      ey += r[c * stride + 1];
      ez += r[c * stride + 2];
    }
    sx -= ex;
    sy -= ey;
    sz -= ez;
  }
  for (int off = 32; off > 0; off >>= 1) {
    sx += __shfl_xor(sx, off);
    sy += __shfl_xor(sy, off);
    sz += __shfl_xor(sz, off);
  }
  if (lane == 0) {
    pos_bar[3 * v + 0] = sx;
    pos_bar[3 * v + 1] = sy;
    pos_bar[3 * v + 2] = sz;
  }
}

int grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_wprep(const WPrepArgs& a, hipStream_t s) {
  if (a.n_paths <= 0) return hipSuccess;
  int maxc = 1;
  for (int t = 0; t < a.n_paths; ++t) maxc = a.cout[t] > maxc ? a.cout[t] : maxc;
  const int64_t per = static_cast<int64_t>(a.nb) * a.c_in * maxc;
  hipLaunchKernelGGL(wprep_kernel, dim3(grid_for(per, 256), a.n_paths), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce_wbar(float* part, int splits, int c_in, int n_paths, int nb, const int64_t* path_off,
                              const int32_t* col0, const int32_t* cout, int ncols, float* out, bool accumulate,
                              hipStream_t s) {
  if (n_paths <= 0) return hipSuccess;
  ReduceWArgs a{};
  a.part = part;
  a.splits = splits;
  a.split_step = 1;
  constexpr int kSeg = 32;
  // many copies (one per persistent workgroup): sum segments of kSeg copies in place, level
  // by level, until at most 2 kSeg remain, so every pass reads its copies with full
  // parallelism and the final pass sums a few per element
  const int64_t stride = static_cast<int64_t>(c_in) * ncols;
  while (a.splits > 2 * kSeg) {
    const int groups = (a.splits + kSeg - 1) / kSeg;
    hipLaunchKernelGGL(segment_sum_kernel, dim3(static_cast<unsigned>((stride + 255) / 256), groups), dim3(256), 0,
                       s, part, a.splits, kSeg, stride, a.split_step);
    a.splits = groups;
    a.split_step *= kSeg;
  }
  a.rows = c_in;
  a.ncols = ncols;
  a.nb = nb;
  a.accumulate = accumulate ? 1 : 0;
  a.out = out;
  int maxc = 1;
  for (int t = 0; t < n_paths && t < kMaxPaths; ++t) {
    a.path_off[t] = path_off[t];
    a.col0[t] = col0[t];
    a.cout[t] = cout[t];
    maxc = cout[t] > maxc ? cout[t] : maxc;
  }
  const int64_t per = static_cast<int64_t>(nb) * c_in * maxc;
  hipLaunchKernelGGL(reduce_wbar_kernel, dim3(grid_for(per, 256), n_paths), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pos_bar(const int32_t* rowptr, const int32_t* s_rowptr, const int32_t* s_slot, const float* rbar,
                          int copies, int64_t n_edges, float* pos_bar, int n_nodes, hipStream_t s) {
  if (n_nodes <= 0) return hipSuccess;
  hipLaunchKernelGGL(pos_bar_kernel, dim3((n_nodes + 3) / 4), dim3(256), 0, s, rowptr, s_rowptr, s_slot, rbar,
                     copies, 3 * n_edges, pos_bar, n_nodes);
  return hipGetLastError();
}

}  // namespace etpc
