// CSR build: stable least-significant-digit radix sort (8-bit digits) of edge ids by
// receiver, then of receiver slots by sender; row pointers by binary search on the
// sorted keys.  Integer work only, bit-exact and deterministic (no atomics whose
// order matters: LDS atomics only count).
//
// The Sobek paper (Sec. 4, the paragraph on layouts and graphs) keeps cached stable
// CSR views, receiver-major and source-major, so every reduction has one owner and
// one fixed order; this builds both views from a COO list.
#include <vector>

#include "kernels.hpp"
#include "sort.hpp"

namespace etpc {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortRounds = 16;                      // items per thread, strided by 256
constexpr int kSortTile = kSortThreads * kSortRounds;
constexpr int kScanThreads = 256;
constexpr int kScanIpt = 8;
constexpr int kScanTile = kScanThreads * kScanIpt;

__global__ void iota_kernel(int32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = static_cast<int32_t>(i);
}

__global__ void copy_kernel(const int32_t* __restrict__ a, int32_t* __restrict__ b, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    b[i] = a[i];
}

// out[i] = a[idx[i]]
__global__ void gather_kernel(const int32_t* __restrict__ a, const int32_t* __restrict__ idx, int32_t* __restrict__ out,
                              int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    out[i] = a[idx[i]];
}

// hist[d * nblk + b] = count of digit d in tile b
__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(const int32_t* __restrict__ keys, int64_t n, int shift,
                                                                 int32_t* __restrict__ hist, int nblk) {
  __shared__ int cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile;
  for (int r = 0; r < kSortRounds; ++r) {
    const int64_t i = base + r * kSortThreads + threadIdx.x;
    if (i < n) atomicAdd(&cnt[(keys[i] >> shift) & 255], 1);
  }
  __syncthreads();
  hist[static_cast<int64_t>(threadIdx.x) * nblk + blockIdx.x] = cnt[threadIdx.x];
}

// Stable scatter: items of a tile are visited in index order (round-major, lane order
// within a round).  Within a wavefront, equal digits are ranked with ballots; waves
// are ordered through per-round digit counts in LDS.
__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(const int32_t* __restrict__ kin,
                                                                    const int32_t* __restrict__ vin,
                                                                    int32_t* __restrict__ kout,
                                                                    int32_t* __restrict__ vout, int64_t n, int shift,
                                                                    const int32_t* __restrict__ hist_scan, int nblk) {
  __shared__ int base_d[256];
  __shared__ int wave_cnt[kSortThreads / 64][256];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  base_d[tid] = hist_scan[static_cast<int64_t>(tid) * nblk + blockIdx.x];
  const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * kSortTile;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kSortRounds; ++r) {
    const int64_t i = tile0 + r * kSortThreads + tid;
    const bool valid = i < n;
    int key = 0, val = 0, d = 0;
    if (valid) {
      key = kin[i];
      val = vin[i];
      d = (key >> shift) & 255;
    }
    for (int t = 0; t < kSortThreads / 64; ++t) wave_cnt[t][tid] = 0;
    __syncthreads();
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wave_cnt[wid][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int off = base_d[d] + rank;
      for (int t = 0; t < wid; ++t) off += wave_cnt[t][d];
      kout[off] = key;
      vout[off] = val;
    }
    __syncthreads();
    int add = 0;
    for (int t = 0; t < kSortThreads / 64; ++t) add += wave_cnt[t][tid];
    base_d[tid] += add;
    __syncthreads();
  }
}

// Exclusive scan, tile level: each block scans kScanTile items and writes its total.
__global__ __launch_bounds__(kScanThreads) void scan_tile_kernel(int32_t* __restrict__ data, int64_t n,
                                                                int32_t* __restrict__ sums) {
  __shared__ int s[kScanThreads];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile + threadIdx.x * kScanIpt;
  int v[kScanIpt];
  int local = 0;
#pragma unroll
  for (int t = 0; t < kScanIpt; ++t) {
    v[t] = (base + t < n) ? data[base + t] : 0;
    local += v[t];
  }
  s[threadIdx.x] = local;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int add = threadIdx.x >= off ? s[threadIdx.x - off] : 0;
    __syncthreads();
    s[threadIdx.x] += add;
    __syncthreads();
  }
  int run = s[threadIdx.x] - local;
#pragma unroll
  for (int t = 0; t < kScanIpt; ++t) {
    if (base + t < n) data[base + t] = run;
    run += v[t];
  }
  if (threadIdx.x == kScanThreads - 1 && sums) sums[blockIdx.x] = s[kScanThreads - 1];
}

__global__ void scan_add_kernel(int32_t* __restrict__ data, int64_t n, const int32_t* __restrict__ sums) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile;
  const int add = sums[blockIdx.x];
  for (int t = threadIdx.x; t < kScanTile; t += blockDim.x)
    if (base + t < n) data[base + t] += add;
}

// rowptr[v] = first index with key >= v (keys sorted ascending), rowptr[n_nodes] = n
__global__ void lower_bound_kernel(const int32_t* __restrict__ keys, int64_t n, int32_t* __restrict__ rowptr,
                                   int n_nodes) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v > n_nodes) return;
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < v)
      lo = mid + 1;
    else
      hi = mid;
  }
  rowptr[v] = static_cast<int32_t>(lo);
}

}  // namespace

int grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

size_t scan_aux_ints(int64_t n) {
  size_t total = 0;
  while (n > kScanTile) {
    n = (n + kScanTile - 1) / kScanTile;
    total += static_cast<size_t>(n);
  }
  return total + 1;
}

hipError_t exclusive_scan(int32_t* data, int64_t n, int32_t* aux, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t nb = (n + kScanTile - 1) / kScanTile;
  if (nb == 1) {
    hipLaunchKernelGGL(scan_tile_kernel, dim3(1), dim3(kScanThreads), 0, s, data, n, static_cast<int32_t*>(nullptr));
    return hipGetLastError();
  }
  hipLaunchKernelGGL(scan_tile_kernel, dim3(static_cast<unsigned>(nb)), dim3(kScanThreads), 0, s, data, n, aux);
  hipError_t e = exclusive_scan(aux, nb, aux + nb, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_add_kernel, dim3(static_cast<unsigned>(nb)), dim3(kScanThreads), 0, s, data, n, aux);
  return hipGetLastError();
}

int radix_passes(int32_t n_nodes) {
  int bits = 0;
  while (bits < 31 && (int64_t(1) << bits) < n_nodes) ++bits;
  return (bits + 7) / 8;
}

size_t sort_scratch_ints(int64_t n) {
  const int64_t nblk = std::max<int64_t>((n + kSortTile - 1) / kSortTile, 1);
  return static_cast<size_t>(256 * nblk) + scan_aux_ints(256 * nblk) + 64;
}

SortBufs make_sort_bufs(int32_t* k0, int32_t* v0, int32_t* k1, int32_t* v1, int32_t* scratch, int64_t n) {
  const int64_t nblk = std::max<int64_t>((n + kSortTile - 1) / kSortTile, 1);
  return SortBufs{k0, v0, k1, v1, scratch, scratch + 256 * nblk};
}

hipError_t launch_copy(const int32_t* a, int32_t* b, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, a, b, n);
  return hipGetLastError();
}

hipError_t launch_lower_bound(const int32_t* keys, int64_t n, int32_t* rowptr, int32_t n_rows, hipStream_t s) {
  hipLaunchKernelGGL(lower_bound_kernel, dim3((n_rows + 1 + 255) / 256), dim3(256), 0, s, keys, n, rowptr, n_rows);
  return hipGetLastError();
}

hipError_t radix_sort(SortBufs& b, int64_t n, int passes, hipStream_t s) {
  const int nblk = static_cast<int>((n + kSortTile - 1) / kSortTile);
  for (int p = 0; p < passes; ++p) {
    const int shift = 8 * p;
    hipLaunchKernelGGL(radix_hist_kernel, dim3(nblk), dim3(kSortThreads), 0, s, b.k0, n, shift, b.hist, nblk);
    hipError_t e = exclusive_scan(b.hist, static_cast<int64_t>(256) * nblk, b.aux, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(nblk), dim3(kSortThreads), 0, s, b.k0, b.v0, b.k1, b.v1, n, shift,
                       b.hist, nblk);
    std::swap(b.k0, b.k1);
    std::swap(b.v0, b.v1);
  }
  return hipGetLastError();
}

namespace {

// key = INT32_MAX - degree, so ascending keys are descending degrees; value = node
__global__ void degree_key_kernel(const int32_t* __restrict__ rowptr, int32_t n, int32_t* __restrict__ key,
                                  int32_t* __restrict__ val) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n) return;
  key[v] = 0x7fffffff - (rowptr[v + 1] - rowptr[v]);
  val[v] = v;
}

// the same over a base sequence: entry k takes node base[k]; rank[base[k]] = k
__global__ void degree_key_base_kernel(const int32_t* __restrict__ rowptr, const int32_t* __restrict__ base, int32_t n,
                                       int32_t* __restrict__ key, int32_t* __restrict__ val,
                                       int32_t* __restrict__ rank) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int v = base[k];
  key[k] = 0x7fffffff - (rowptr[v + 1] - rowptr[v]);
  val[k] = v;
  rank[v] = k;
}

// second key: the window of the node each entry now holds (by its index, or by its
// position in the base sequence)
__global__ void window_key_kernel(const int32_t* __restrict__ val, const int32_t* __restrict__ rank, int32_t n,
                                  int32_t window, int32_t* __restrict__ key) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) key[t] = (rank ? rank[val[t]] : val[t]) / window;
}

// Morton (Z-order) key of a position: 10 bits per axis of the cell of the point in a
// 1024^3 grid over the box (periodic: the coordinate wrapped into [0, L)) or over the
// bounding box lo[3] / ext[3] found by bbox_dev_kernel.
__device__ inline uint32_t spread_bits10(uint32_t v) {
  v &= 0x3ffu;
  v = (v | (v << 16)) & 0x030000ffu;
  v = (v | (v << 8)) & 0x0300f00fu;
  v = (v | (v << 4)) & 0x030c30c3u;
  v = (v | (v << 2)) & 0x09249249u;
  return v;
}

// one workgroup: lo[3], ext[3] of the points (ext >= a tiny positive floor)
__global__ __launch_bounds__(1024) void bbox_dev_kernel(const float* __restrict__ pos, int32_t n,
                                                        float* __restrict__ box6) {
  __shared__ float red[6][1024];
  float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  for (int64_t i = threadIdx.x; i < n; i += 1024)
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const float v = pos[3 * i + a];
      mn[a] = fminf(mn[a], v);
      mx[a] = fmaxf(mx[a], v);
    }
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    red[a][threadIdx.x] = mn[a];
    red[3 + a][threadIdx.x] = mx[a];
  }
  __syncthreads();
  for (int h = 512; h > 0; h >>= 1) {
    if (threadIdx.x < h)
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        red[a][threadIdx.x] = fminf(red[a][threadIdx.x], red[a][threadIdx.x + h]);
        red[3 + a][threadIdx.x] = fmaxf(red[3 + a][threadIdx.x], red[3 + a][threadIdx.x + h]);
      }
    __syncthreads();
  }
  if (threadIdx.x < 3) {
    const int a = threadIdx.x;
    box6[a] = red[a][0];
    box6[3 + a] = fmaxf(red[3 + a][0] - red[a][0], 1e-30f);
  }
}

struct MortonFrame {
  float box[3];       // periodic box lengths (periodic = 1)
  int32_t periodic;
};

__global__ void morton_key_kernel(const float* __restrict__ pos, int32_t n, const MortonFrame f,
                                  const float* __restrict__ box6, int32_t* __restrict__ key,
                                  int32_t* __restrict__ val) {
  // each operation rounded on its own (no fused multiply-add), so the cell of a point is
  // the one that plain IEEE single-precision arithmetic gives
#pragma clang fp contract(off)
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n) return;
  uint32_t code = 0;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const float p = pos[3 * v + a];
    float t;
    if (f.periodic) {
      const float L = f.box[a];
      t = (p - L * floorf(p / L)) / L;
    } else {
      t = (p - box6[a]) / box6[3 + a];
    }
    const float c = fminf(fmaxf(t * 1024.f, 0.f), 1023.f);
    code |= spread_bits10(static_cast<uint32_t>(c)) << a;
  }
  key[v] = static_cast<int32_t>(code);
  val[v] = v;
}

}  // namespace

size_t degree_order_bytes(int32_t n) {
  const size_t a = (static_cast<size_t>(n) + 63) & ~size_t(63);
  return sizeof(int32_t) * (5 * a + sort_scratch_ints(n));
}

etpc_status degree_order_impl(int32_t n, const int32_t* rowptr, int32_t window, const int32_t* base_order,
                              int32_t* order, void* ws, hipStream_t s) {
  if (n == 0) return ETPC_OK;
  const size_t a = (static_cast<size_t>(n) + 63) & ~size_t(63);
  int32_t* base = static_cast<int32_t*>(ws);
  int32_t* rank = base + 4 * a;
  SortBufs b = make_sort_bufs(base, base + a, base + 2 * a, base + 3 * a, base + 5 * a, n);
  if (base_order)
    hipLaunchKernelGGL(degree_key_base_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, rowptr, base_order, n, b.k0,
                       b.v0, rank);
  else
    hipLaunchKernelGGL(degree_key_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, rowptr, n, b.k0, b.v0);
  // a stable LSD sort over all four key bytes: ties keep increasing node index (or the
  // base sequence)
  ETPC_HIP(radix_sort(b, n, 4, s));
  if (window > 0 && window < n) {
    // then stably by window (radix sort keys must be non-negative: v / window is):
    // window-major, heaviest first inside each window
    hipLaunchKernelGGL(window_key_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, b.v0,
                       base_order ? rank : nullptr, n, window, b.k0);
    ETPC_HIP(radix_sort(b, n, radix_passes((n + window - 1) / window), s));
  }
  ETPC_HIP(launch_copy(b.v0, order, n, s));
  return ETPC_OK;
}

size_t spatial_order_bytes(int32_t n) {
  const size_t a = (static_cast<size_t>(n) + 63) & ~size_t(63);
  return sizeof(int32_t) * (4 * a + sort_scratch_ints(n) + 64);
}

etpc_status spatial_order_impl(int32_t n, const float* pos, const float* box, int32_t* order, void* ws,
                               hipStream_t s) {
  if (n == 0) return ETPC_OK;
  const size_t a = (static_cast<size_t>(n) + 63) & ~size_t(63);
  int32_t* base = static_cast<int32_t*>(ws);
  float* box6 = reinterpret_cast<float*>(base + 4 * a);
  SortBufs b = make_sort_bufs(base, base + a, base + 2 * a, base + 3 * a, base + 4 * a + 64, n);
  MortonFrame f{};
  if (box) {
    f.periodic = 1;
    for (int d = 0; d < 3; ++d) f.box[d] = box[d];
  } else {
    hipLaunchKernelGGL(bbox_dev_kernel, dim3(1), dim3(1024), 0, s, pos, n, box6);
  }
  hipLaunchKernelGGL(morton_key_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, pos, n, f, box6, b.k0, b.v0);
  // 30-bit keys: four stable digit passes, ties in increasing node index
  ETPC_HIP(radix_sort(b, n, 4, s));
  ETPC_HIP(launch_copy(b.v0, order, n, s));
  return ETPC_OK;
}

namespace {

__device__ int g_graph_error;

__global__ void validate_rowptr_kernel(const int32_t* __restrict__ rp, int n, int64_t e, int code) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v > n) return;
  bool bad = false;
  if (v == 0 && rp[0] != 0) bad = true;
  if (v == n && rp[n] != e) bad = true;
  if (v < n && rp[v + 1] < rp[v]) bad = true;
  if (bad) atomicMax(&g_graph_error, code);
}

// receiver slots: sender in range, no self loop, and the sender view holds this slot
__global__ void validate_slots_kernel(const etpc_graph g) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= g.n_nodes) return;
  for (int64_t e = g.rowptr[i]; e < g.rowptr[i + 1]; ++e) {
    const int j = g.col[e];
    if (j < 0 || j >= g.n_nodes) {
      atomicMax(&g_graph_error, 3);
      return;
    }
    if (j == i) {
      atomicMax(&g_graph_error, 4);
      return;
    }
    int64_t lo = g.s_rowptr[j], hi = g.s_rowptr[j + 1];
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (g.s_slot[mid] < e)
        lo = mid + 1;
      else
        hi = mid;
    }
    if (lo >= g.s_rowptr[j + 1] || g.s_slot[lo] != e || g.s_col[lo] != i) {
      atomicMax(&g_graph_error, 5);
      return;
    }
  }
}

// sender rows: strictly increasing slots in range
// order with windows of w positions: every entry in range, counted once per occurrence
// (count[], zeroed by the caller), and the degrees of each window's entries
// non-increasing (ties in any order: index order or a base order such as the spatial one)
__global__ void validate_order_kernel(const int32_t* __restrict__ order, const int32_t* __restrict__ rp, int n,
                                      int w, int32_t* __restrict__ count) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int v = order[k];
  if (v < 0 || v >= n) {
    atomicMax(&g_graph_error, 7);
    return;
  }
  atomicAdd(&count[v], 1);
  if (k + 1 < n && (k + 1) / w == k / w) {
    const int u = order[k + 1];
    if (u < 0 || u >= n) return;   // reported by thread k + 1
    const int dv = rp[v + 1] - rp[v], du = rp[u + 1] - rp[u];
    if (dv < du) atomicMax(&g_graph_error, 7);
  }
}

// every node counted exactly once: the order is a permutation
__global__ void validate_count_kernel(const int32_t* __restrict__ count, int n) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < n && count[v] != 1) atomicMax(&g_graph_error, 7);
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < n) p[v] = 0;
}

__global__ void validate_sender_rows_kernel(const etpc_graph g) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= g.n_nodes) return;
  for (int64_t k = g.s_rowptr[j]; k < g.s_rowptr[j + 1]; ++k) {
    const int64_t sl = g.s_slot[k];
    if (sl < 0 || sl >= g.n_edges || (k > g.s_rowptr[j] && g.s_slot[k - 1] >= sl)) {
      atomicMax(&g_graph_error, 6);
      return;
    }
  }
}

}  // namespace

size_t csr_workspace_bytes(int32_t n_nodes, int64_t n_edges) {
  const int64_t nblk = (n_edges + kSortTile - 1) / kSortTile;
  const int64_t hist = 256 * std::max<int64_t>(nblk, 1);
  // five E-sized arrays and the histogram, each start rounded up to 64 ints, then the scan scratch
  const size_t ints = 5 * static_cast<size_t>(n_edges) + static_cast<size_t>(hist) + scan_aux_ints(hist) + 7 * 64;
  (void)n_nodes;
  return ints * sizeof(int32_t) + 256;
}

etpc_status csr_build_impl(int32_t n_nodes, int64_t n_edges, const int32_t* src, const int32_t* dst, int32_t* rowptr,
                           int32_t* col, int32_t* eid, int32_t* s_rowptr, int32_t* s_col, int32_t* s_slot, void* ws,
                           hipStream_t s) {
  const int64_t E = n_edges;
  const int threads = 256;
  auto align = [](size_t x) { return (x + 63) & ~size_t(63); };
  int32_t* base = static_cast<int32_t*>(ws);
  size_t o = 0;
  SortBufs b{};
  b.k0 = base + o; o = align(o + E);
  b.v0 = base + o; o = align(o + E);
  b.k1 = base + o; o = align(o + E);
  b.v1 = base + o; o = align(o + E);
  int32_t* sorted_dst = base + o; o = align(o + E);
  const int64_t nblk = (E + kSortTile - 1) / kSortTile;
  b.hist = base + o; o = align(o + 256 * std::max<int64_t>(nblk, 1));
  b.aux = base + o;
  const int passes = radix_passes(n_nodes);
  if (E > 0) {
    // receiver view
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, dst, b.k0, E);
    hipLaunchKernelGGL(iota_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, b.v0, E);
    ETPC_HIP(radix_sort(b, E, passes, s));
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, b.k0, sorted_dst, E);
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, b.v0, eid, E);
    hipLaunchKernelGGL(gather_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, src, eid, col, E);
  }
  hipLaunchKernelGGL(lower_bound_kernel, dim3((n_nodes + 1 + threads - 1) / threads), dim3(threads), 0, s, sorted_dst,
                     E, rowptr, n_nodes);
  if (E > 0) {
    // sender view: sort receiver slots by their sender, stably
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, col, b.k0, E);
    hipLaunchKernelGGL(iota_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, b.v0, E);
    ETPC_HIP(radix_sort(b, E, passes, s));
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, b.v0, s_slot, E);
    hipLaunchKernelGGL(gather_kernel, dim3(grid_for(E, threads)), dim3(threads), 0, s, sorted_dst, s_slot, s_col, E);
  }
  hipLaunchKernelGGL(lower_bound_kernel, dim3((n_nodes + 1 + threads - 1) / threads), dim3(threads), 0, s,
                     E > 0 ? b.k0 : sorted_dst, E, s_rowptr, n_nodes);
  ETPC_HIP(hipGetLastError());
  return ETPC_OK;
}

etpc_status graph_validate_impl(const etpc_graph& g, hipStream_t s) {
  const int zero = 0;
  ETPC_HIP(hipMemcpyToSymbolAsync(HIP_SYMBOL(g_graph_error), &zero, sizeof(int), 0, hipMemcpyHostToDevice, s));
  const int threads = 256;
  const int blocks = (g.n_nodes + 1 + threads - 1) / threads;
  hipLaunchKernelGGL(validate_rowptr_kernel, dim3(blocks), dim3(threads), 0, s, g.rowptr, g.n_nodes, g.n_edges, 1);
  hipLaunchKernelGGL(validate_rowptr_kernel, dim3(blocks), dim3(threads), 0, s, g.s_rowptr, g.n_nodes, g.n_edges, 2);
  ETPC_HIP(hipGetLastError());
  int err = 0;
  ETPC_HIP(hipMemcpyFromSymbolAsync(&err, HIP_SYMBOL(g_graph_error), sizeof(int), 0, hipMemcpyDeviceToHost, s));
  ETPC_HIP(hipStreamSynchronize(s));
  if (err == 0) {
    hipLaunchKernelGGL(validate_sender_rows_kernel, dim3(blocks), dim3(threads), 0, s, g);
    hipLaunchKernelGGL(validate_slots_kernel, dim3(blocks), dim3(threads), 0, s, g);
    int32_t* count = nullptr;
    if ((g.s_order != nullptr || g.r_order != nullptr) && g.n_nodes > 0)
      ETPC_HIP(hipMalloc(&count, sizeof(int32_t) * static_cast<size_t>(g.n_nodes)));
    const int32_t* orders[2] = {g.s_order, g.r_order};
    const int32_t* rps[2] = {g.s_rowptr, g.rowptr};
    const int windows[2] = {static_cast<int>(ETPC_SEND_ORDER_WINDOW), static_cast<int>(ETPC_RECV_ORDER_WINDOW)};
    for (int o = 0; o < 2; ++o) {
      if (orders[o] == nullptr || g.n_nodes == 0) continue;
      hipLaunchKernelGGL(zero_i32_kernel, dim3(blocks), dim3(threads), 0, s, count, g.n_nodes);
      hipLaunchKernelGGL(validate_order_kernel, dim3(blocks), dim3(threads), 0, s, orders[o], rps[o], g.n_nodes,
                         windows[o], count);
      hipLaunchKernelGGL(validate_count_kernel, dim3(blocks), dim3(threads), 0, s, count, g.n_nodes);
    }
    const hipError_t launched = hipGetLastError();
    if (count != nullptr) {
      const hipError_t synced = hipStreamSynchronize(s);
      ETPC_HIP(hipFree(count));
      ETPC_HIP(synced);
    }
    ETPC_HIP(launched);
    ETPC_HIP(hipMemcpyFromSymbolAsync(&err, HIP_SYMBOL(g_graph_error), sizeof(int), 0, hipMemcpyDeviceToHost, s));
    ETPC_HIP(hipStreamSynchronize(s));
  }
  static const char* what[] = {"",
                               "receiver rowptr is not a monotone 0..E sequence",
                               "sender rowptr is not a monotone 0..E sequence",
                               "receiver col out of range",
                               "self loop (sender == receiver)",
                               "sender view does not hold a receiver slot (or s_col mismatch)",
                               "sender row slots out of range or not strictly increasing",
                               "s_order or r_order is not a permutation with decreasing degree within windows"};
  if (err != 0) ETPC_FAIL(ETPC_ERR_GRAPH, what[err]);
  return ETPC_OK;
}

}  // namespace etpc
