// Graph preparation: the radius graph of a point set, built on the GPU with a cell list.
//
// The convolution runs on radius graphs (an edge joins two atoms closer than the cutoff;
// at fixed density |E| grows as |V| rho r_c^3: Sobek paper, Sec. 3, the paragraph on
// edge growth), and the wrapper prepares the graph from the positions (Sec. 4, the
// implementation paragraph).  The edge test is fixed exactly, in float32 with every
// product and sum rounded on its own, so the edge set is a function of the float32
// positions alone and does not depend on the cell grid:
//   d_a = p_j,a - p_i,a;  periodic: d_a -= L_a * rint(d_a * (1/L_a));
//   edge j -> i  iff  0 < (d_x^2 + d_y^2) + d_z^2 < r_c^2   (i != j).
// Steps: bounding box (open boundary), cell keys, stable radix sort of atoms by cell,
// cell row pointers, per-atom neighbour counts over the 27 surrounding cells, a scan,
// the fill, then the canonical (receiver, sender) order: rows come out in receiver order,
// so when no row exceeds 256 edges one wavefront per row sorts its senders; otherwise two
// stable radix sorts (by sender, then by receiver) order the whole list.  Cells are at least r_c (1 + 2^-10) wide,
// so every pair inside the cutoff lies in adjacent cells whatever the rounding of the
// cell index.
#include <algorithm>
#include <cstdint>
#include <cmath>
#include <string>

#include "kernels.hpp"
#include "profile.hpp"
#include "sort.hpp"

namespace etpc {
namespace {

constexpr int kBoxBlocks = 256;
constexpr int kThreads = 256;

struct CellGrid {
  int32_t n[3];
  int32_t periodic;
  float lo[3];      // open: bounding-box minimum
  float inv_w[3];   // cells per unit length
  float L[3];       // periodic box
  float invL[3];    // float32 1 / L
  float c2;         // float32 r_c * r_c
};

// partial[b] = (min x, min y, min z, max x, max y, max z, any non-finite, -)
__global__ __launch_bounds__(kThreads) void bbox_kernel(const float* __restrict__ pos, int32_t n,
                                                        float* __restrict__ partial) {
  __shared__ float red[6][kThreads];
  __shared__ int bad_any;
  if (threadIdx.x == 0) bad_any = 0;
  float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  int bad = 0;
  for (int64_t i = blockIdx.x * int64_t(kThreads) + threadIdx.x; i < n; i += int64_t(gridDim.x) * kThreads) {
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const float v = pos[3 * i + a];
      if (!isfinite(v)) bad = 1;
      mn[a] = fminf(mn[a], v);
      mx[a] = fmaxf(mx[a], v);
    }
  }
  __syncthreads();
  if (bad) atomicOr(&bad_any, 1);
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    red[a][threadIdx.x] = mn[a];
    red[3 + a][threadIdx.x] = mx[a];
  }
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) {
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        red[a][threadIdx.x] = fminf(red[a][threadIdx.x], red[a][threadIdx.x + h]);
        red[3 + a][threadIdx.x] = fmaxf(red[3 + a][threadIdx.x], red[3 + a][threadIdx.x + h]);
      }
    }
    __syncthreads();
  }
  if (threadIdx.x < 6) partial[8 * blockIdx.x + threadIdx.x] = red[threadIdx.x][0];
  if (threadIdx.x == 6) partial[8 * blockIdx.x + 6] = bad_any ? 1.f : 0.f;
  if (threadIdx.x == 7) partial[8 * blockIdx.x + 7] = 0.f;
}

__device__ inline int cell_coord(float p, int a, const CellGrid& g) {
  float q;
  if (g.periodic)
    q = p - g.L[a] * floorf(p * g.invL[a]);
  else
    q = p - g.lo[a];
  int c = static_cast<int>(floorf(q * g.inv_w[a]));
  return min(max(c, 0), g.n[a] - 1);
}

// keys[i] = cell of atom i, vals[i] = i
__global__ void cell_key_kernel(const float* __restrict__ pos, int32_t n, const CellGrid g, int32_t* __restrict__ keys,
                                int32_t* __restrict__ vals) {
  const int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (i >= n) return;
  const int cx = cell_coord(pos[3 * i], 0, g);
  const int cy = cell_coord(pos[3 * i + 1], 1, g);
  const int cz = cell_coord(pos[3 * i + 2], 2, g);
  keys[i] = (cz * g.n[1] + cy) * g.n[0] + cx;
  vals[i] = static_cast<int32_t>(i);
}

// spos[k] = (x, y, z, id) of the k-th atom in cell order (original coordinates)
__global__ void gather_pos_kernel(const float* __restrict__ pos, const int32_t* __restrict__ ids, int32_t n,
                                  float4* __restrict__ spos) {
  const int64_t k = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (k >= n) return;
  const int32_t i = ids[k];
  spos[k] = make_float4(pos[3 * i], pos[3 * i + 1], pos[3 * i + 2], __int_as_float(i));
}

// The exact edge test; no fused multiply-add, so it matches a float32 evaluation that
// rounds every operation.
__device__ inline bool in_range(const float4 pi, const float4 pj, const CellGrid& g) {
#pragma clang fp contract(off)
  float dx = pj.x - pi.x, dy = pj.y - pi.y, dz = pj.z - pi.z;
  if (g.periodic) {
    dx = dx - g.L[0] * rintf(dx * g.invL[0]);
    dy = dy - g.L[1] * rintf(dy * g.invL[1]);
    dz = dz - g.L[2] * rintf(dz * g.invL[2]);
  }
  const float r2 = (dx * dx + dy * dy) + dz * dz;
  return r2 > 0.f && r2 < g.c2;
}

// Cells visited along one axis around cell c: c-1..c+1 (wrapped when periodic with at
// least three cells), every cell when a periodic axis has fewer than three, clipped to
// the grid when open.  Returns the count; the cells go to out[0..count).
__device__ inline int axis_cells(int c, int a, const CellGrid& g, int* out) {
  const int n = g.n[a];
  int k = 0;
  if (g.periodic) {
    if (n >= 3) {
      out[0] = c == 0 ? n - 1 : c - 1;
      out[1] = c;
      out[2] = c == n - 1 ? 0 : c + 1;
      return 3;
    }
    for (int t = 0; t < n; ++t) out[k++] = t;
    return k;
  }
  for (int t = max(c - 1, 0); t <= min(c + 1, n - 1); ++t) out[k++] = t;
  return k;
}

// One thread per atom (in cell order).  FILL = false: counts[i] = number of neighbours,
// counts[n] = 0, total[0] += sum, total[1] = max(total[1], count).  FILL = true: writes the neighbours of i at
// rowptr[i]..rowptr[i+1] as (src = j, dst = i).
template <bool FILL>
__global__ __launch_bounds__(kThreads) void neighbour_kernel(const float4* __restrict__ spos,
                                                             const int32_t* __restrict__ cell_of,
                                                             const int32_t* __restrict__ cellptr, int32_t n,
                                                             const CellGrid g, int32_t* __restrict__ counts,
                                                             unsigned long long* __restrict__ total,
                                                             int32_t* __restrict__ e_src, int32_t* __restrict__ e_dst) {
  const int64_t k = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (!FILL && k == 0) counts[n] = 0;
  int cnt = 0;
  if (k < n) {
    const float4 pi = spos[k];
    const int32_t i = __float_as_int(pi.w);
    const int key = cell_of[k];
    const int cx = key % g.n[0];
    const int cy = (key / g.n[0]) % g.n[1];
    const int cz = key / (g.n[0] * g.n[1]);
    int xs[3], ys[3], zs[3];
    const int nx = axis_cells(cx, 0, g, xs), ny = axis_cells(cy, 1, g, ys), nz = axis_cells(cz, 2, g, zs);
    int32_t out = FILL ? counts[i] : 0;
    for (int a = 0; a < nz; ++a)
      for (int b = 0; b < ny; ++b)
        for (int c = 0; c < nx; ++c) {
          const int cell = (zs[a] * g.n[1] + ys[b]) * g.n[0] + xs[c];
          const int t1 = cellptr[cell + 1];
          for (int t = cellptr[cell]; t < t1; ++t) {
            const float4 pj = spos[t];
            const int32_t j = __float_as_int(pj.w);
            if (j == i || !in_range(pi, pj, g)) continue;
            if (FILL) {
              e_src[out] = j;
              e_dst[out] = i;
              ++out;
            } else {
              ++cnt;
            }
          }
        }
    if (!FILL) counts[i] = cnt;
  }
  if (!FILL) {
    // one integer atomic per wavefront; the sum does not depend on their order
    unsigned long long v = static_cast<unsigned long long>(cnt), m = v;
    for (int off = 32; off > 0; off >>= 1) {
      v += __shfl_down(v, off, 64);
      m = max(m, __shfl_down(m, off, 64));
    }
    if ((threadIdx.x & 63) == 0 && v) {
      atomicAdd(total, v);
      atomicMax(total + 1, m);
    }
  }
}

__global__ void zero_u64_kernel(unsigned long long* p) {
  p[0] = 0ull;
  p[1] = 0ull;
}

// Sorts each row of at most 64 K senders ascending in place: one wavefront per row, each
// lane holding K values (element r * 64 + lane in register r), a bitonic network whose
// partners at distance j < 64 are other lanes (shuffles) and at j >= 64 other registers
// of the same lane.  Padding holds INT32_MAX and sorts to the end.
constexpr int kRowSortRows = 4;   // rows (wavefronts) per 256-thread workgroup
template <int K>
__global__ __launch_bounds__(256) void row_sort_kernel(const int32_t* __restrict__ rowptr, int32_t n,
                                                      int32_t* __restrict__ src) {
  constexpr int M = 64 * K;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowSortRows + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;   // whole wavefronts only
  const int32_t b = rowptr[row], len = rowptr[row + 1] - b;
  int32_t v[K];
#pragma unroll
  for (int r = 0; r < K; ++r) v[r] = r * 64 + lane < len ? src[b + r * 64 + lane] : INT32_MAX;
#pragma unroll
  for (int k = 2; k <= M; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 64) {
        const int rj = j >> 6;
#pragma unroll
        for (int r = 0; r < K; ++r)
          if ((r & rj) == 0) {
            const bool ascending = ((r * 64 + lane) & k) == 0;
            const int32_t lo = min(v[r], v[r | rj]), hi = max(v[r], v[r | rj]);
            v[r] = ascending ? lo : hi;
            v[r | rj] = ascending ? hi : lo;
          }
      } else {
#pragma unroll
        for (int r = 0; r < K; ++r) {
          const int32_t other = __shfl_xor(v[r], j, 64);
          const bool lower = (lane & j) == 0, ascending = ((r * 64 + lane) & k) == 0;
          v[r] = (lower == ascending) ? min(v[r], other) : max(v[r], other);
        }
      }
    }
#pragma unroll
  for (int r = 0; r < K; ++r)
    if (r * 64 + lane < len) src[b + r * 64 + lane] = v[r];
}

struct RadiusLayout {
  float* partial;
  unsigned long long* total;
  int32_t *ak0, *av0, *ak1, *av1, *asort;   // atom sort buffers + scratch
  float4* spos;
  int32_t* cellptr;
  int32_t *counts, *scan_aux;
  int32_t *ek0, *ev0, *ek1, *ev1, *esort;   // edge sort buffers + scratch
  size_t bytes;
};

int64_t max_cells(int32_t n) { return 2 * static_cast<int64_t>(n) + 64; }

RadiusLayout carve(void* base, int32_t n, int64_t max_edges) {
  RadiusLayout L{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) -> void* {
    off = (off + 255) & ~size_t(255);
    void* p = b ? b + off : nullptr;
    off += bytes;
    return p;
  };
  const size_t N = static_cast<size_t>(n), E = static_cast<size_t>(max_edges);
  L.partial = static_cast<float*>(take(sizeof(float) * 8 * kBoxBlocks));
  L.total = static_cast<unsigned long long*>(take(2 * sizeof(unsigned long long)));   // edges, max degree
  L.ak0 = static_cast<int32_t*>(take(4 * N));
  L.av0 = static_cast<int32_t*>(take(4 * N));
  L.ak1 = static_cast<int32_t*>(take(4 * N));
  L.av1 = static_cast<int32_t*>(take(4 * N));
  L.asort = static_cast<int32_t*>(take(4 * sort_scratch_ints(n)));
  L.spos = static_cast<float4*>(take(16 * N));
  L.cellptr = static_cast<int32_t*>(take(4 * (static_cast<size_t>(max_cells(n)) + 1)));
  L.counts = static_cast<int32_t*>(take(4 * (N + 1)));
  L.scan_aux = static_cast<int32_t*>(take(4 * scan_aux_ints(n + 1)));
  L.ek0 = static_cast<int32_t*>(take(4 * E));
  L.ev0 = static_cast<int32_t*>(take(4 * E));
  L.ek1 = static_cast<int32_t*>(take(4 * E));
  L.ev1 = static_cast<int32_t*>(take(4 * E));
  L.esort = static_cast<int32_t*>(take(4 * sort_scratch_ints(max_edges)));
  L.bytes = off + 256;
  return L;
}

// Cell counts along each axis for extents ext[a] and minimum cell width w_min, widened
// until the grid has at most `cap` cells.
void grid_dims(const double ext[3], double w_min, int64_t cap, int32_t n_out[3]) {
  double w = w_min;
  for (;;) {
    int64_t prod = 1;
    int64_t na[3];
    for (int a = 0; a < 3; ++a) {
      const double f = std::floor(ext[a] / w);
      na[a] = f < 1.0 ? 1 : (f > 1048576.0 ? 1048576 : static_cast<int64_t>(f));
      prod = std::min<int64_t>(prod * na[a], int64_t(1) << 62);
    }
    if (prod <= cap) {
      for (int a = 0; a < 3; ++a) n_out[a] = static_cast<int32_t>(na[a]);
      return;
    }
    w *= 1.25;
  }
}

}  // namespace

size_t radius_workspace_bytes(int32_t n_nodes, int64_t max_edges) {
  return carve(nullptr, n_nodes, max_edges).bytes;
}

etpc_status radius_graph_impl(int32_t n, const float* pos, float cutoff, const float* box, int64_t max_edges,
                              int32_t* src, int32_t* dst, int64_t* n_edges, void* ws, hipStream_t s) {
  const RadiusLayout W = carve(ws, n, max_edges);
  CellGrid g{};
  g.periodic = box != nullptr;
  g.c2 = cutoff * cutoff;
  const double margin_w = static_cast<double>(cutoff) * (1.0 + 1.0 / 1024.0);

  // bounding box (also the non-finite check)
  const int nbb = std::max(1, std::min(kBoxBlocks, (n + kThreads - 1) / kThreads));
  {
    ::etpc::ProfScope ps(ETPC_KIND_PREP, s);
    hipLaunchKernelGGL(bbox_kernel, dim3(nbb), dim3(kThreads), 0, s, pos, n, W.partial);
    ETPC_HIP(hipGetLastError());
  }
  float part[8 * kBoxBlocks];
  ETPC_HIP(hipMemcpyAsync(part, W.partial, sizeof(float) * 8 * nbb, hipMemcpyDeviceToHost, s));
  ETPC_HIP(hipStreamSynchronize(s));
  float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  for (int b = 0; b < nbb; ++b) {
    if (part[8 * b + 6] != 0.f) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "positions hold a non-finite value");
    for (int a = 0; a < 3; ++a) {
      mn[a] = std::min(mn[a], part[8 * b + a]);
      mx[a] = std::max(mx[a], part[8 * b + 3 + a]);
    }
  }
  double ext[3];
  double ext_max = 0.0;
  for (int a = 0; a < 3; ++a) {
    if (g.periodic) {
      g.L[a] = box[a];
      g.invL[a] = 1.0f / box[a];
      ext[a] = box[a];
    } else {
      g.lo[a] = mn[a];
      ext[a] = static_cast<double>(mx[a]) - static_cast<double>(mn[a]);
    }
    ext_max = std::max(ext_max, std::max(std::fabs(static_cast<double>(mn[a])), std::fabs(static_cast<double>(mx[a]))));
    ext_max = std::max(ext_max, ext[a]);
  }
  // rounding of the cell index is a few ulps of the coordinates; the margin covers it
  grid_dims(ext, margin_w + ext_max * (1.0 / 65536.0), max_cells(n), g.n);
  for (int a = 0; a < 3; ++a) g.inv_w[a] = ext[a] > 0.0 ? static_cast<float>(g.n[a] / ext[a]) : 0.f;
  const int32_t ncells = g.n[0] * g.n[1] * g.n[2];

  // one thread per atom, no stride loop: the grid covers every atom (n < 2^30)
  const unsigned nb = static_cast<unsigned>((static_cast<int64_t>(n) + kThreads - 1) / kThreads);
  SortBufs ab = make_sort_bufs(W.ak0, W.av0, W.ak1, W.av1, W.asort, n);
  {
    ::etpc::ProfScope ps(ETPC_KIND_PREP, s);
    hipLaunchKernelGGL(cell_key_kernel, dim3(nb), dim3(kThreads), 0, s, pos, n, g, ab.k0, ab.v0);
    ETPC_HIP(hipGetLastError());
    ETPC_HIP(radix_sort(ab, n, radix_passes(ncells), s));
    hipLaunchKernelGGL(gather_pos_kernel, dim3(nb), dim3(kThreads), 0, s, pos, ab.v0, n, W.spos);
    ETPC_HIP(hipGetLastError());
    ETPC_HIP(launch_lower_bound(ab.k0, n, W.cellptr, ncells, s));
    hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, s, W.total);
    hipLaunchKernelGGL(neighbour_kernel<false>, dim3(nb), dim3(kThreads), 0, s, W.spos, ab.k0, W.cellptr, n, g,
                       W.counts, W.total, static_cast<int32_t*>(nullptr), static_cast<int32_t*>(nullptr));
    ETPC_HIP(hipGetLastError());
  }
  unsigned long long counters[2] = {0ull, 0ull};
  ETPC_HIP(hipMemcpyAsync(counters, W.total, sizeof(counters), hipMemcpyDeviceToHost, s));
  ETPC_HIP(hipStreamSynchronize(s));
  const unsigned long long total = counters[0], max_degree = counters[1];
  *n_edges = static_cast<int64_t>(total);
  if (total >= (1ull << 31)) ETPC_FAIL(ETPC_ERR_OVERFLOW, "the radius graph has 2^31 edges or more");
  if (static_cast<int64_t>(total) > max_edges)
    ETPC_FAIL(ETPC_ERR_CAPACITY, "max_edges = " + std::to_string(max_edges) + " is below the " +
                                     std::to_string(total) + " edges of the radius graph (returned in *n_edges)");
  const int64_t E = static_cast<int64_t>(total);
  const int epasses = radix_passes(n);
  SortBufs eb = make_sort_bufs(W.ek0, W.ev0, W.ek1, W.ev1, W.esort, E);
  {
    ::etpc::ProfScope ps(ETPC_KIND_PREP, s);
    ETPC_HIP(exclusive_scan(W.counts, static_cast<int64_t>(n) + 1, W.scan_aux, s));
    if (max_degree <= 256) {
      // rows already in receiver order: fill the outputs and sort each row's senders
      hipLaunchKernelGGL(neighbour_kernel<true>, dim3(nb), dim3(kThreads), 0, s, W.spos, ab.k0, W.cellptr, n, g,
                         W.counts, W.total, src, dst);
      ETPC_HIP(hipGetLastError());
      const unsigned rb = static_cast<unsigned>((static_cast<int64_t>(n) + kRowSortRows - 1) / kRowSortRows);
      if (E > 0) {
        if (max_degree <= 64)
          hipLaunchKernelGGL(row_sort_kernel<1>, dim3(rb), dim3(256), 0, s, W.counts, n, src);
        else if (max_degree <= 128)
          hipLaunchKernelGGL(row_sort_kernel<2>, dim3(rb), dim3(256), 0, s, W.counts, n, src);
        else
          hipLaunchKernelGGL(row_sort_kernel<4>, dim3(rb), dim3(256), 0, s, W.counts, n, src);
      }
      ETPC_HIP(hipGetLastError());
      return ETPC_OK;
    }
    hipLaunchKernelGGL(neighbour_kernel<true>, dim3(nb), dim3(kThreads), 0, s, W.spos, ab.k0, W.cellptr, n, g,
                       W.counts, W.total, eb.k0, eb.v0);
    ETPC_HIP(hipGetLastError());
    if (E > 0) {
      // (k0, v0) = (src, dst) grouped by receiver: sort stably by sender, then by receiver
      ETPC_HIP(radix_sort(eb, E, epasses, s));
      std::swap(eb.k0, eb.v0);
      std::swap(eb.k1, eb.v1);
      ETPC_HIP(radix_sort(eb, E, epasses, s));
      ETPC_HIP(launch_copy(eb.k0, dst, E, s));
      ETPC_HIP(launch_copy(eb.v0, src, E, s));
    }
  }
  return ETPC_OK;
}

}  // namespace etpc
