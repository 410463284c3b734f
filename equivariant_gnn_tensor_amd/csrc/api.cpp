// C ABI: argument validation, workspace carving, chunk scheduling and launches.
//
// Schedules (one ordered unit of the caller's stream, deterministic for a given workspace
// and lane setting; the per-path launches of a pass fork onto up to two lanes and the
// node-side GEMMs onto the post stream, see lanes.hpp):
//  forward uvw  -- per output group g (largest first), per receiver chunk: one receiver
//                  traversal per path of g builds the receiver state S_g (Sobek paper,
//                  Sec. 4, Eq. 33) in one of two S sets, then one MFMA GEMM m_g = S_g W_g
//                  writes the output rows (Eq. 34-35) on the post stream while the next
//                  group's traversals fill the other set.
//  forward uvu  -- one receiver traversal per path writes the output block (Eq. 7, 17).
//  backward uvw -- a pipeline over (sender chunk, input block) items, two buffer sets:
//                  Xt = x W (GEMM, if positions are wanted; for the next item on the post
//                  stream), one sender traversal per path of the block (P state and the
//                  edge position adjoint), then x_bar = P W^T and W_bar = x^T P (GEMMs,
//                  split-K with a fixed-order reduction) on the post stream; finally
//                  pos_bar from the edge adjoints by a segment sum over both CSR views
//                  (Eq. 18-22).
//  backward uvu -- one sender traversal per path (x_bar, W_bar partials, edge adjoint).
//  double backward -- the directional program of Eq. 23-31 / 37-39 assembled from the
//                  same traversals in tangent mode plus the same GEMMs.
#include <algorithm>
#include <cmath>
#include <optional>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.hpp"
#include "lanes.hpp"
#include "plan.hpp"
#include "profile.hpp"

namespace etpc {
size_t csr_workspace_bytes(int32_t n_nodes, int64_t n_edges);
etpc_status csr_build_impl(int32_t n_nodes, int64_t n_edges, const int32_t* src, const int32_t* dst, int32_t* rowptr,
                           int32_t* col, int32_t* eid, int32_t* s_rowptr, int32_t* s_col, int32_t* s_slot, void* ws,
                           hipStream_t s);
etpc_status graph_validate_impl(const etpc_graph& g, hipStream_t s);
size_t degree_order_bytes(int32_t n);
etpc_status degree_order_impl(int32_t n, const int32_t* rowptr, int32_t window, const int32_t* base_order,
                              int32_t* order, void* ws, hipStream_t s);
size_t spatial_order_bytes(int32_t n);
etpc_status spatial_order_impl(int32_t n, const float* pos, const float* box, int32_t* order, void* ws,
                               hipStream_t s);
size_t radius_workspace_bytes(int32_t n_nodes, int64_t max_edges);
etpc_status radius_graph_impl(int32_t n, const float* pos, float cutoff, const float* box, int64_t max_edges,
                              int32_t* src, int32_t* dst, int64_t* n_edges, void* ws, hipStream_t s);
etpc_status layout_convert_impl(const std::vector<etpc_irrep>& irreps, int direction, int32_t n_rows,
                                const float* in, float* out, hipStream_t s);
}  // namespace etpc

namespace {

using namespace etpc;

constexpr int kMaxSplits = 32;

struct Carver {
  char* base = nullptr;
  size_t off = 0;
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

// Lanes per edge slot: the channel count rounded up to a power of two (whole waves above
// 64), at least min_cp.  The sender traversals take min_cp = 16: their per-edge lane sums
// are DPP row sums, and their 4x4x1 matrix-core updates combine groups of four lanes,
// which must belong to one edge slot.
int lane_width(int c, int* ntiles, int min_cp = 1) {
  if (c > kWave) {
    *ntiles = (c + kWave - 1) / kWave;
    return kWave;
  }
  int cp = min_cp;
  while (cp < c) cp <<= 1;
  *ntiles = 1;
  return cp;
}

// Concurrent lanes of a pass (see lanes.hpp).  uvw: paths round-robin over the lanes;
// uvu: one lane per input block (backward: x_bar accumulates per block) or per output
// block (forward: z accumulates per block).  Each lane owns a copy of the edge adjoint:
// the workspace holds rbar_slots copies (one per lane the plan allows); a call uses
// rbar_lanes of them (one when the call is too small to gain from lanes).
int count_blocks(const etpc_plan_s* p, bool by_in) {
  const auto& groups = by_in ? p->by_in : p->by_out;
  int used = 0;
  for (const auto& gr : groups) used += gr.empty() ? 0 : 1;
  return used;
}
int rbar_slots(const etpc_plan_s* p) {
  const int units = p->mode == ETPC_UVW ? static_cast<int>(p->paths.size()) : count_blocks(p, true);
  return std::max(1, std::min(std::min(p->lanes, kLanes), units));
}
// Below about 2^16 edge-channels a pass's launches take a few microseconds each, less
// than a fork and join of side streams costs, so such calls stay on one lane.
constexpr int64_t kLaneMinWork = int64_t(1) << 16;
int lane_cap(const etpc_plan_s* p, const etpc_graph* g) {
  int64_t cmax = 1;
  for (const auto& b : p->in) cmax = std::max<int64_t>(cmax, b.mul);
  for (const auto& b : p->out) cmax = std::max<int64_t>(cmax, b.mul);
  return g->n_edges * cmax < kLaneMinWork ? 1 : std::max(1, std::min(p->lanes, kLanes));
}
int rbar_lanes(const etpc_plan_s* p, const etpc_graph* g) { return std::min(rbar_slots(p), lane_cap(p, g)); }
// lane of each block for n lanes (blocks without paths get lane 0, unused)
std::vector<int> block_lanes(const etpc_plan_s* p, bool by_in, int n) {
  const auto& groups = by_in ? p->by_in : p->by_out;
  std::vector<int> lane(groups.size(), 0);
  int used = 0;
  for (size_t k = 0; k < groups.size(); ++k)
    if (!groups[k].empty()) lane[k] = (used++) % n;
  return lane;
}

// ---------------------------------------------------------------- per-plan derived sizes
struct Derived {
  int64_t max_s = 0;                 // max_g o_g * D_g (uvw forward state floats per receiver)
  std::vector<int64_t> group_d;      // D_g
  std::vector<int64_t> block_ncols;  // sum over paths of block k of B * C_out
  std::vector<std::vector<int32_t>> block_col0;
  int64_t max_state = 0;             // max_k (2l_k+1) * ncols_k
  int64_t max_wcat = 0;              // max_k C_in_k * ncols_k
  int64_t max_zrow = 0;              // max_g o_g * C_out_g (channel GEMM output floats per receiver)
  int64_t max_xrow = 0;              // max_k i_k * C_in_k (x_bar GEMM output floats per sender)
};

Derived derive(const etpc_plan_s* p) {
  Derived d;
  d.group_d.assign(p->out.size(), 0);
  for (size_t g = 0; g < p->out.size(); ++g) {
    int64_t D = 0;
    for (int q : p->by_out[g]) D += static_cast<int64_t>(p->n_basis) * p->paths[q].c_in;
    d.group_d[g] = D;
    d.max_s = std::max<int64_t>(d.max_s, D * (2 * p->out[g].l + 1));
    d.max_zrow = std::max<int64_t>(d.max_zrow, static_cast<int64_t>(2 * p->out[g].l + 1) * p->out[g].mul);
  }
  d.block_ncols.assign(p->in.size(), 0);
  d.block_col0.assign(p->in.size(), {});
  for (size_t k = 0; k < p->in.size(); ++k) {
    int64_t n = 0;
    for (int q : p->by_in[k]) {
      d.block_col0[k].push_back(static_cast<int32_t>(n));
      n += static_cast<int64_t>(p->n_basis) * p->paths[q].c_out;
    }
    d.block_ncols[k] = n;
    d.max_state = std::max<int64_t>(d.max_state, n * (2 * p->in[k].l + 1));
    d.max_wcat = std::max<int64_t>(d.max_wcat, n * p->in[k].mul);
    d.max_xrow = std::max<int64_t>(d.max_xrow, static_cast<int64_t>(2 * p->in[k].l + 1) * p->in[k].mul);
  }
  return d;
}

// Workgroups a split-K GEMM aims for (split count = this / output tiles, at least 256 rows
// of K per split).
#ifndef ETPC_GEMM_TARGET_WG
#define ETPC_GEMM_TARGET_WG 1024
#endif
constexpr int64_t kGemmTargetWg = ETPC_GEMM_TARGET_WG;

int pick_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int64_t sp = (kGemmTargetWg + tiles - 1) / tiles;
  sp = std::min<int64_t>(sp, (K + 255) / 256);
  sp = std::max<int64_t>(1, std::min<int64_t>(sp, kMaxSplits));
  return static_cast<int>(sp);
}

// ---------------------------------------------------------------- workspace layouts
// split-K partial sets kept for the long-K channel / x_bar GEMMs
#ifndef ETPC_GEMM_SPLIT_SLOTS
#define ETPC_GEMM_SPLIT_SLOTS 8
#endif
constexpr int kGemmSplits = ETPC_GEMM_SPLIT_SLOTS;

// Up to two sets of the buffers the node-side GEMMs read (S forward; Xt, P and the
// re-laid-out weights backward): work items alternate between them, so one item's GEMMs
// can run on the post stream while the next item's traversals fill the other set.
constexpr int kSets = 2;

// How a uvw pass uses its workspace.  The node-side state (forward: the receiver state S
// of an output group, Eq. 33; backward: Xt and P of an input block) lives in `nsets`
// buffers of `cap` floats each, and the pass runs as a list of work items (make_items)
// that each fit one buffer.
//  fast (the workspace holds every node's state of the largest group / block): one item
//    per group or block, two buffer sets, one edge-adjoint copy per lane, kGemmSplits
//    split-K partial slots.
//  bounded (a smaller workspace, e.g. one sized by a scratch budget): a group's or
//    block's paths are split into subsets whose state for every node fits a buffer, so
//    every traversal launch still covers all nodes (Sobek Sec. 4 keeps complete output
//    groups inside the scratch budget); only when one path's state for every node does
//    not fit are the nodes chunked, one path at a time.  Two buffer sets while no node
//    chunking is needed, else one; one edge-adjoint copy per lane only while those take
//    at most an eighth of the workspace; split-K partials in a quarter of a buffer (the
//    GEMMs take fewer splits to fit).
struct Sched {
  bool bounded = false;
  int nsets = kSets;
  int rbar_copies = 1;
};

// Above this many bytes per copy the edge adjoint keeps one copy (the traversals that write
// it then run on one lane): such passes have long launches whose tails a second lane barely
// fills, and a second copy would add 12 B per edge to a workspace that is otherwise flat in E.
constexpr int64_t kRbarLaneMaxBytes = int64_t(64) << 20;
Sched fast_sched(const etpc_plan_s* p, int64_t n_edges) {
  Sched s;
  s.rbar_copies = 12 * n_edges > kRbarLaneMaxBytes ? 1 : rbar_slots(p);
  return s;
}

// One work item of a uvw pass: nodes [n0, n0 + nn) of output group (forward) or input
// block (backward) `blk`, and its paths [t0, t1) (positions in by_out[blk] / by_in[blk]).
// Their state columns [col0, col0 + ncols) of the group's or block's column space
// ((path, q, channel) in plan order) sit in the item's buffer from column 0.
struct Item {
  int64_t n0;
  int32_t nn;
  int32_t blk, t0, t1;
  int64_t col0, ncols;
};

// state columns of each path of a group (forward: B C_in) or block (backward: B C_out)
std::vector<int64_t> path_cols(const etpc_plan_s* p, int blk, bool fwd) {
  const auto& paths = fwd ? p->by_out[blk] : p->by_in[blk];
  std::vector<int64_t> c(paths.size());
  for (size_t t = 0; t < paths.size(); ++t) {
    const PathInfo& pi = p->paths[paths[t]];
    c[t] = static_cast<int64_t>(p->n_basis) * (fwd ? pi.c_in : pi.c_out);
  }
  return c;
}

// rows per node of a group's (forward, 2 l_out + 1) or block's (backward, 2 l_in + 1) state
int state_rows(const etpc_plan_s* p, int blk, bool fwd) { return 2 * (fwd ? p->out[blk].l : p->in[blk].l) + 1; }

std::vector<int> group_order(const etpc_plan_s* p, const Derived& d);
std::vector<int> block_order(const etpc_plan_s* p, const Derived& d);

std::vector<Item> make_items(const etpc_plan_s* p, const Derived& d, bool fwd, int64_t n, int64_t cap, bool bounded) {
  std::vector<Item> items;
  if (n <= 0) return items;
  for (const int blk : fwd ? group_order(p, d) : block_order(p, d)) {
    const std::vector<int64_t> cols = path_cols(p, blk, fwd);
    const int np = static_cast<int>(cols.size());
    const int64_t m = state_rows(p, blk, fwd);
    int64_t total = 0, widest = 0;
    for (const int64_t c : cols) {
      total += c;
      widest = std::max(widest, c);
    }
    if (!bounded || n * m * total <= cap) {
      items.push_back(Item{0, static_cast<int32_t>(n), blk, 0, np, 0, total});
      continue;
    }
    if (n * m * widest <= cap) {   // complete node ranges for subsets of the paths
      int64_t col0 = 0;
      for (int t0 = 0; t0 < np;) {
        int t1 = t0;
        int64_t c = 0;
        while (t1 < np && n * m * (c + cols[t1]) <= cap) c += cols[t1++];
        items.push_back(Item{0, static_cast<int32_t>(n), blk, t0, t1, col0, c});
        col0 += c;
        t0 = t1;
      }
      continue;
    }
    const int64_t nn = std::max<int64_t>(1, cap / (m * widest));   // node chunks of single paths
    for (int64_t n0 = 0; n0 < n; n0 += nn) {
      int64_t col0 = 0;
      for (int t = 0; t < np; ++t) {
        items.push_back(Item{n0, static_cast<int32_t>(std::min(nn, n - n0)), blk, t, t + 1, col0, cols[t]});
        col0 += cols[t];
      }
    }
  }
  return items;
}

// smallest buffer of a bounded schedule: one node of the widest path of any group / block
int64_t min_cap(const etpc_plan_s* p, bool fwd, bool bwd) {
  int64_t c = 0;
  if (fwd)
    for (size_t g = 0; g < p->out.size(); ++g)
      for (const int64_t w : path_cols(p, static_cast<int>(g), true)) c = std::max(c, w * state_rows(p, g, true));
  if (bwd)
    for (size_t k = 0; k < p->in.size(); ++k)
      for (const int64_t w : path_cols(p, static_cast<int>(k), false)) c = std::max(c, w * state_rows(p, k, false));
  return c;
}

// buffer that holds every node's state of the largest group / block (the fast schedule)
int64_t full_cap(const Derived& d, int64_t n, bool fwd, bool bwd) {
  return n * std::max(fwd ? d.max_s : int64_t(0), bwd ? d.max_state : int64_t(0));
}

struct FwdLayout {
  float* S[kSets] = {};
  float* part = nullptr;
  int64_t part_cap = 0;
  int nsets = kSets;
  int64_t cap = 0;
};
// n_nodes: the graph's node count (the fast schedule's split-K partials cover all of them)
void fwd_layout(const etpc_plan_s* p, const Derived& d, int64_t n_nodes, int64_t cap, const Sched& sch, Carver& c,
                FwdLayout& L) {
  L.nsets = sch.nsets;
  L.cap = cap;
  if (p->mode == ETPC_UVW) {
    for (int b = 0; b < sch.nsets; ++b) L.S[b] = c.take<float>(static_cast<size_t>(cap));
    L.part_cap = sch.bounded ? cap / 4 : kGemmSplits * n_nodes * d.max_zrow;
    L.part = c.take<float>(static_cast<size_t>(L.part_cap));
  }
}

struct BwdLayout {
  float *rbar = nullptr, *wpart = nullptr;
  float *wcat[kSets] = {}, *wt[kSets] = {}, *wt2[kSets] = {};
  float *xt[kSets] = {}, *P[kSets] = {}, *Pd[kSets] = {};
  float* xpart = nullptr;
  int64_t xpart_cap = 0;
  int64_t wpart_cap = 0;    // uvw: floats of W_bar split-K partials (one or two operand sets)
  int64_t wpart_lane = 0;   // uvu: floats of W_bar partials per lane
  int nsets = kSets;
  int rbar_copies = 1;
  int64_t cap = 0;
};
// flags: pos = edge adjoint (sch.rbar_copies copies) + Xt; p = plain P state; tan = tangent state; wbar = W_bar
// partials (two sets when wbar2); wt2 = second transposed weight (for w_dot).  uvw: cap = floats per state
// buffer; uvu: cap = the persistent grid size.
void bwd_layout(const etpc_plan_s* p, const Derived& d, int64_t n_nodes, int64_t n_edges, int64_t cap,
                const Sched& sch, bool pos, bool need_p, bool tan, bool wbar, bool wbar2, bool xbar, bool wt2,
                Carver& c, BwdLayout& L) {
  L.nsets = sch.nsets;
  L.rbar_copies = sch.rbar_copies;
  L.cap = cap;
  if (p->mode == ETPC_UVW) {
    if (pos) L.rbar = c.take<float>(static_cast<size_t>(3 * n_edges * sch.rbar_copies));
    for (int b = 0; b < sch.nsets; ++b) {
      if (pos) L.wcat[b] = c.take<float>(static_cast<size_t>(d.max_wcat));
      if (xbar) L.wt[b] = c.take<float>(static_cast<size_t>(d.max_wcat));
      if (wt2) L.wt2[b] = c.take<float>(static_cast<size_t>(d.max_wcat));
    }
    if (wbar) {
      // split-K partial tiles of W_bar: fast, as many splits as wbar_gemm picks for a whole
      // block; bounded, four sets of the largest block or 32 of its widest path, whichever
      // is more (an item of one path has few output tiles and needs more splits to fill the
      // chip; wbar_gemm fits its splits to this room)
      int64_t need = 0;
      for (size_t k = 0; k < p->in.size(); ++k) {
        if (p->by_in[k].empty()) continue;
        const int ni = 2 * p->in[k].l + 1;
        const int64_t blockw = static_cast<int64_t>(p->in[k].mul) * d.block_ncols[k];
        if (sch.bounded) {
          int64_t widest = 0;
          for (const int64_t w : path_cols(p, static_cast<int>(k), false)) widest = std::max(widest, w);
          need = std::max<int64_t>(need, std::max<int64_t>(4 * blockw, 32 * p->in[k].mul * widest));
        } else {
          need = std::max<int64_t>(
              need, pick_splits(p->in[k].mul, d.block_ncols[k], std::max<int64_t>(n_nodes, 1) * ni) * blockw);
        }
      }
      L.wpart_cap = (wbar2 ? 2 : 1) * need;
      L.wpart = c.take<float>(static_cast<size_t>(L.wpart_cap));
    }
    for (int b = 0; b < sch.nsets; ++b) {
      if (pos) L.xt[b] = c.take<float>(static_cast<size_t>(cap));
      if (need_p) L.P[b] = c.take<float>(static_cast<size_t>(cap));
      if (tan) L.Pd[b] = c.take<float>(static_cast<size_t>(cap));
    }
    if (xbar) {
      L.xpart_cap = sch.bounded ? cap / 4 : kGemmSplits * n_nodes * d.max_xrow;
      L.xpart = c.take<float>(static_cast<size_t>(L.xpart_cap));
    }
  } else {
    if (pos) L.rbar = c.take<float>(static_cast<size_t>(3 * n_edges * sch.rbar_copies));
    int64_t maxbc = 0;
    for (auto& q : p->paths) maxbc = std::max<int64_t>(maxbc, static_cast<int64_t>(p->n_basis) * q.c_in);
    L.wpart_lane = cap * maxbc;   // cap = uvu grid size here; one partial set per lane
    if (wbar) L.wpart = c.take<float>(static_cast<size_t>(L.wpart_lane * rbar_slots(p)));
  }
}

// Persistent grid of the uvu sender traversal (W_bar partials: one per workgroup).  At
// three resident waves per SIMD (1536 two-wave workgroups) the channelwise workload's
// backward traversals take 14.5 / 12.9 / 11.8 ms per step with 2048 / 3072 / 4608
// workgroups (3-4 senders each at 4608, so the launch ends with a short tail).
#ifndef ETPC_UVU_GRID
#define ETPC_UVU_GRID 4608
#endif
constexpr int kUvuGrid = ETPC_UVU_GRID;

size_t fwd_bytes(const etpc_plan_s* p, const Derived& d, int64_t n_nodes, int64_t cap, const Sched& sch) {
  Carver c;
  FwdLayout L;
  fwd_layout(p, d, n_nodes, cap, sch, c, L);
  return c.off;
}

size_t bwd_bytes(const etpc_plan_s* p, const Derived& d, int64_t n_nodes, int64_t n_edges, int64_t cap,
                 const Sched& sch) {
  Carver c;
  BwdLayout L;
  bwd_layout(p, d, n_nodes, n_edges, p->mode == ETPC_UVW ? cap : kUvuGrid, sch, true, true, false, true, false, true,
             false, c, L);
  return c.off;
}

size_t dbl_bytes(const etpc_plan_s* p, const Derived& d, int64_t n_nodes, int64_t n_edges, int64_t cap,
                 const Sched& sch) {
  Carver c;
  BwdLayout L;
  bwd_layout(p, d, n_nodes, n_edges, p->mode == ETPC_UVW ? cap : kUvuGrid, sch, true, true, true, true, true, true,
             true, c, L);   // every output
  return std::max(c.off, fwd_bytes(p, d, n_nodes, cap, sch));
}

// The schedule and state buffer size of a uvw pass given ws_bytes of workspace:
// bytes_of(cap, sched) is the pass's layout size; fwd / bwd say which state the pass keeps.
// The fast schedule when every node fits at once; else the bounded one with the largest
// buffer that fits (two sets while that needs no node chunks); cap = -1 when not even
// one node of one path fits.  uvu passes keep no node state (cap unused).
template <class F>
void choose_schedule(const etpc_plan_s* p, const Derived& d, bool fwd, bool bwd, int64_t n_nodes, int64_t n_edges,
                     size_t ws_bytes, F bytes_of, Sched* sch, int64_t* cap) {
  const Sched f = fast_sched(p, n_edges);
  const int64_t cfull = p->mode == ETPC_UVW ? full_cap(d, n_nodes, fwd, bwd) : 0;
  if (n_nodes <= 0 || bytes_of(cfull, f) <= ws_bytes) {
    *sch = f;
    *cap = cfull;
    return;
  }
  Sched b;
  b.bounded = true;
  const int slots = rbar_slots(p);
  const size_t all = static_cast<size_t>(3 * sizeof(float)) * static_cast<size_t>(n_edges) * slots;
  b.rbar_copies = (slots > 1 && all <= ws_bytes / 8) ? slots : 1;
  if (p->mode != ETPC_UVW) {
    b.nsets = 1;
    *sch = b;
    *cap = bytes_of(0, b) <= ws_bytes ? 0 : -1;
    return;
  }
  // largest buffer in [lo, hi] that fits (bytes_of grows with cap)
  auto largest = [&](const Sched& sc) -> int64_t {
    int64_t lo = min_cap(p, fwd, bwd), hi = cfull;
    if (bytes_of(lo, sc) > ws_bytes) return -1;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo + 1) / 2;
      if (bytes_of(mid, sc) <= ws_bytes)
        lo = mid;
      else
        hi = mid - 1;
    }
    return lo;
  };
  // two sets while each set still holds the widest path's state for every node
  int64_t need_all = 0;
  if (fwd)
    for (size_t g = 0; g < p->out.size(); ++g)
      for (const int64_t w : path_cols(p, static_cast<int>(g), true))
        need_all = std::max(need_all, n_nodes * w * state_rows(p, g, true));
  if (bwd)
    for (size_t k = 0; k < p->in.size(); ++k)
      for (const int64_t w : path_cols(p, static_cast<int>(k), false))
        need_all = std::max(need_all, n_nodes * w * state_rows(p, k, false));
  b.nsets = 2;
  int64_t c2 = largest(b);
  if (c2 >= need_all) {
    *sch = b;
    *cap = c2;
    return;
  }
  b.nsets = 1;
  *sch = b;
  *cap = largest(b);
}

RowMap plain(int64_t ld) { return make_rowmap(ld, 0, 1); }
RowMap irmul(int32_t m, int64_t width, int64_t mul) { return make_rowmap(width, mul, m); }


bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool map4(const RowMap& m) { return m.s1 % 4 == 0 && (m.div == 1 || m.s2 % 4 == 0); }

void set_vec4(GemmArgs& ga) {
  ga.vec4 = (aligned16(ga.A) && map4(ga.amap) && aligned16(ga.B) && ga.ldb % 4 == 0) ? 1 : 0;
}

// Launch ga (final destination C / cmap / beta).  When K is long relative to the number
// of output tiles, split K across workgroups into `part` (capacity part_cap floats) and
// sum the partial tiles in a fixed order into C.
etpc_status gemm_auto(GemmArgs ga, float* part, int64_t part_cap, int max_splits, int kind, hipStream_t s) {
  set_vec4(ga);
  int sp = std::min(pick_splits(ga.M, ga.N, ga.K), max_splits);
  const int64_t mn = static_cast<int64_t>(ga.M) * ga.N;
  if (part == nullptr || mn <= 0) sp = 1;
  while (sp > 1 && static_cast<int64_t>(sp) * mn > part_cap) --sp;
  if (sp <= 1) {
    ga.k_split = ga.K;
    ga.c_split_stride = 0;
    ETPC_LAUNCH(kind, launch_gemm(ga, 1, s));
    return ETPC_OK;
  }
  int64_t ks = (ga.K + sp - 1) / sp;
  ks = (ks + kGemmBK - 1) / kGemmBK * kGemmBK;
  sp = static_cast<int>((ga.K + ks - 1) / ks);
  float* C = ga.C;
  const RowMap cmap = ga.cmap;
  const bool beta = ga.beta != 0;
  ga.C = part;
  ga.cmap = plain(ga.N);
  ga.beta = 0;
  ga.k_split = static_cast<int32_t>(ks);
  ga.c_split_stride = mn;
  ETPC_LAUNCH(kind, launch_gemm(ga, sp, s));
  ETPC_LAUNCH(ETPC_KIND_AUX, launch_splitk_reduce(part, sp, ga.M, ga.N, C, cmap, beta, s));
  return ETPC_OK;
}

// ---------------------------------------------------------------- validation
etpc_status check_common(const etpc_plan_s* p, const etpc_graph* g) {
  if (p == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null plan");
  if (g == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null graph");
  if (g->n_nodes < 0 || g->n_edges < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative graph size");
  if (g->n_edges >= (int64_t(1) << 31)) ETPC_FAIL(ETPC_ERR_OVERFLOW, "n_edges must be < 2^31");
  if (static_cast<int64_t>(g->n_nodes) * 7 >= (int64_t(1) << 31))
    ETPC_FAIL(ETPC_ERR_OVERFLOW, "n_nodes * 7 must be < 2^31");
  if (g->n_nodes > 0 && (g->rowptr == nullptr || g->s_rowptr == nullptr))
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null row pointers");
  if (g->n_edges > 0 && (g->col == nullptr || g->s_col == nullptr || g->s_slot == nullptr))
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null CSR index arrays");
  return ETPC_OK;
}

etpc_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need > 0 && ws == nullptr) ETPC_FAIL(ETPC_ERR_WORKSPACE, "workspace is null but the pass needs one");
  if (ws_bytes < need)
    ETPC_FAIL(ETPC_ERR_WORKSPACE, "workspace too small: need at least " + std::to_string(need) + " bytes");
  return ETPC_OK;
}

etpc_status check_channels_bwd(const etpc_plan_s* p) {
  for (auto& q : p->paths) {
    const int c = p->mode == ETPC_UVW ? q.c_out : q.c_in;
    if (c > 64 * 4) ETPC_FAIL(ETPC_ERR_UNSUPPORTED, "backward supports at most 256 channels per block");
  }
  return ETPC_OK;
}

// ---------------------------------------------------------------- forward pieces
// zero output blocks that receive no path
hipError_t zero_unreached(const etpc_plan_s* p, float* z, int32_t n, hipStream_t s) {
  bool any = false;
  for (size_t g = 0; g < p->out.size(); ++g) any |= p->by_out[g].empty();
  if (!any) return hipSuccess;
  return launch_fill(z, static_cast<int64_t>(n) * p->z_dim, 0.f, s);
}

hipError_t zero_unreached_in(const etpc_plan_s* p, float* x, int32_t n, hipStream_t s) {
  bool any = false;
  for (size_t k = 0; k < p->in.size(); ++k) any |= p->by_in[k].empty();
  if (!any) return hipSuccess;
  return launch_fill(x, static_cast<int64_t>(n) * p->x_dim, 0.f, s);
}

// Waves that split one node's edges inside a traversal workgroup (1, 2 or 4).  A launch
// over few nodes has one workgroup per node and at most one wave per SIMD, each walking
// its whole edge list in series (latency bound: a 128-atom cell); splitting the edges over
// more waves shortens that walk.  Used while the launch stays under 1024 waves, the mean
// degree gives each wave at least 12 edges, and the state the waves exchange at the end
// (`states` accumulators of (2 l + 1) x B floats per lane and channel tile) fits kSplitMaxLds.
constexpr int64_t kSplitMaxWaves = 1024;   // 4096 measured slower on 2048-node launches
// The exchange buffer stays at 24 KB so that, with the edge record (up to ~20 KB) and the
// edge-adjoint partials (up to 12 KB), a workgroup stays inside the default 64 KB of LDS.
constexpr int64_t kSplitMaxLds = 24 * 1024;
int edge_parts(int nodes, int ntiles, const etpc_graph* g, int l, int nb, int states) {
  const int64_t deg = g->n_nodes > 0 ? g->n_edges / g->n_nodes : 0;
  const int64_t nbp = nb <= 8 ? 8 : 16;
  int np = 1;
  while (np < 4 && ntiles * np * 2 <= 4 && static_cast<int64_t>(nodes) * ntiles * np * 2 <= kSplitMaxWaves &&
         deg >= 12 * np * 2 && int64_t(ntiles) * 64 * (2 * l + 1) * nbp * states * 4 <= kSplitMaxLds)
    np *= 2;
  return np;
}

// Output groups with paths, by decreasing channel-GEMM work per node (o C_out D_g), ties
// in plan order.
std::vector<int> group_order(const etpc_plan_s* p, const Derived& d) {
  std::vector<int> order;
  for (size_t gi = 0; gi < p->out.size(); ++gi)
    if (!p->by_out[gi].empty()) order.push_back(static_cast<int>(gi));
  auto work = [&](int gi) { return int64_t(2 * p->out[gi].l + 1) * p->out[gi].mul * d.group_d[gi]; };
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return work(a) > work(b); });
  return order;
}

// Input blocks with paths, by increasing node-GEMM work per node ((2l+1) C_in ncols), ties
// in plan order: the first block's Xt product, which no traversal hides, is the smallest,
// and the largest products run beside the traversals of the blocks after them (workload 2
// 2.62-2.63 -> 2.58-2.59 ms against the decreasing order; the pass then ends on the
// largest block's x_bar / W_bar products, which cost less than the first Xt they replace).
std::vector<int> block_order(const etpc_plan_s* p, const Derived& d) {
  std::vector<int> order;
  for (size_t k = 0; k < p->in.size(); ++k)
    if (!p->by_in[k].empty()) order.push_back(static_cast<int>(k));
  auto work = [&](int k) { return int64_t(2 * p->in[k].l + 1) * p->in[k].mul * d.block_ncols[k]; };
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return work(a) < work(b); });
  return order;
}

// Whether work enqueued on s is being captured into a HIP graph.  Passes keep their
// lanes forked across work items only outside capture: under capture they join the lanes
// at every item, the form whose captured graphs are tested to replay bit-identically.
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

// One uvw forward evaluation into z (beta: accumulate into z).  With tangent, the
// receiver traversal builds dS along pos_dot.  xin / win select the operands.
// nl: concurrent lanes the call may use (lane_cap, or 1 to stay on the caller's stream).
etpc_status fwd_uvw_run(const etpc_plan_s* p, const Derived& d, const etpc_graph* g, const float* xin,
                        const float* pos, const float* pos_dot, const float* win, float* z, bool beta, bool tangent,
                        const FwdLayout& L, const Sched& sch, int nl, hipStream_t s) {
  const GeomParams geom = p->geom();
  const int32_t N = g->n_nodes;
  // the channel GEMM of one item runs on the post stream while the next item's
  // traversals fill the other S set; the largest groups go first, so they overlap most.
  // With the post stream the lanes stay forked for the whole pass: a lane goes on to the
  // next item's paths as soon as its own are done (only the GEMM waits for every lane),
  // and waits for the GEMM that last read the S set it is about to fill.
  PostStream post(s, nl > 1);
  ETPC_HIP(post.status());
  // Bounded schedules (many small items) join the lanes per item: keeping them measured
  // 6% slower there (workload 2 at a 256 MiB budget) and neutral elsewhere.
  const bool keep = post.enabled() && !capturing(s) && !sch.bounded;
  std::optional<LaneGroup> pass_lanes;
  if (keep) {
    pass_lanes.emplace(s, nl);
    ETPC_HIP(pass_lanes->status());
  }
  int set = 0, t_glob = 0;
  for (const Item& it : make_items(p, d, true, N, L.cap, sch.bounded)) {
    const int gi = it.blk;
    const auto& paths = p->by_out[gi];
    const int no = 2 * p->out[gi].l + 1;
    const int c_out = p->out[gi].mul;
    const int nrecv = it.nn;
    // the item's paths fill disjoint column ranges of S: concurrent lanes
    std::optional<LaneGroup> item_lanes;
    if (!keep) {
      ETPC_HIP(post.wait_slot(set));
      item_lanes.emplace(s, std::min(it.t1 - it.t0, nl));
      ETPC_HIP(item_lanes->status());
    }
    LaneGroup& lanes = keep ? *pass_lanes : *item_lanes;
    unsigned waited = 0;   // kept lanes that already wait for this item's S set
    int64_t col0 = 0;
    for (int t = 0; t < it.t1; ++t) {
      const PathInfo& pi = p->paths[paths[t]];
      const int64_t cols = static_cast<int64_t>(p->n_basis) * pi.c_in;
      if (t < it.t0) {
        col0 += cols;
        continue;
      }
      FwdUvwArgs a{};
      a.rowptr = g->rowptr;
      a.col = g->col;
      a.pos = pos;
      a.pos_dot = pos_dot;
      a.x = xin;
      a.S = L.S[set];
      a.recv0 = static_cast<int32_t>(it.n0);
      a.order = (g->r_order != nullptr && it.n0 == 0 && nrecv == g->n_nodes) ? g->r_order : nullptr;
      a.x_dim = static_cast<int32_t>(p->x_dim);
      a.xoff = static_cast<int32_t>(p->xoff[pi.in_block]);
      int ntiles = 1;
      a.cp = lane_width(pi.c_in, &ntiles, 4);   // 4-lane matrix-core blocks never mix edges
      a.c_in = pi.c_in;
      a.ls = pi.l_sh;
      a.s_row_stride = it.ncols;
      a.s_col0 = static_cast<int32_t>(col0 - it.col0);
      // one workgroup per (receiver, channel tile): the tiles are separate workgroups
      a.nparts = edge_parts(nrecv * ntiles, 1, g, pi.l_out, p->n_basis, 1);
      a.g = geom;
      a.cg = pi.cgf;
      const int lane = keep ? t_glob++ % nl : t - it.t0;
      const hipStream_t ls = lanes.lane(lane);
      if (keep && !(waited & (1u << lane))) {
        ETPC_HIP(post.wait_slot_on(ls, set));
        waited |= 1u << lane;
      }
      ETPC_LAUNCH_ON(ETPC_KIND_FWD_TRAVERSE, ls, launch_fwd_uvw(a, tangent, pi.l_in, pi.l_out, nrecv, ntiles, ls));
      col0 += cols;
    }
    if (keep)
      ETPC_HIP(lanes.signal(post.stream()));
    else
      ETPC_HIP(lanes.finish());
    ETPC_HIP(post.follow());
    // z rows of the item's receivers (+)= S W over the item's paths: the first path subset
    // of a node range writes (unless the caller accumulates), later ones add
    GemmArgs ga{};
    ga.lowp = p->gemm_precision;
    ga.A = L.S[set];
    ga.amap = plain(it.ncols);
    ga.a_mcontig = 0;
    ga.B = win + p->paths[paths[it.t0]].w_off;
    ga.ldb = c_out;
    ga.C = z + it.n0 * p->z_dim + p->zoff[gi];
    ga.cmap = irmul(no, p->z_dim, c_out);
    ga.beta = (beta || it.t0 > 0) ? 1 : 0;
    ga.M = nrecv * no;
    ga.N = c_out;
    ga.K = static_cast<int32_t>(it.ncols);
    etpc_status st = gemm_auto(ga, L.part, L.part_cap, kGemmSplits, ETPC_KIND_CHANNEL_GEMM, post.stream());
    if (st != ETPC_OK) return st;
    ETPC_HIP(post.mark(set));
    if (L.nsets > 1) set ^= 1;
  }
  if (keep) ETPC_HIP(pass_lanes->finish());
  ETPC_HIP(post.finish());
  return ETPC_OK;
}

etpc_status fwd_uvu_run(const etpc_plan_s* p, const etpc_graph* g, const float* xin, const float* pos,
                        const float* pos_dot, const float* win, float* z, bool beta, bool tangent, int nlanes,
                        hipStream_t s) {
  const GeomParams geom = p->geom();
  std::vector<int> seen(p->out.size(), 0);
  const int nl = std::max(1, std::min(nlanes, count_blocks(p, false)));
  const std::vector<int> lane_of = block_lanes(p, false, nl);   // z accumulates per output block
  LaneGroup lanes(s, nl);
  ETPC_HIP(lanes.status());
  for (const PathInfo& pi : p->paths) {
    FwdUvuArgs a{};
    a.rowptr = g->rowptr;
    a.col = g->col;
    a.pos = pos;
    a.pos_dot = pos_dot;
    a.x = xin;
    a.w = win + pi.w_off;
    a.z = z;
    a.order = g->r_order;
    a.x_dim = static_cast<int32_t>(p->x_dim);
    a.xoff = static_cast<int32_t>(p->xoff[pi.in_block]);
    a.z_dim = static_cast<int32_t>(p->z_dim);
    a.zoff = static_cast<int32_t>(p->zoff[pi.out_block]);
    int ntiles = 1;
    a.cp = lane_width(pi.c_in, &ntiles, 4);   // 4-lane matrix-core blocks never mix edges
    a.c = pi.c_in;
    a.ls = pi.l_sh;
    a.accumulate = (beta || seen[pi.out_block]) ? 1 : 0;
    a.g = geom;
    a.cg = pi.cgf;
    const hipStream_t ls = lanes.lane(lane_of[pi.out_block]);
    ETPC_LAUNCH_ON(ETPC_KIND_FWD_TRAVERSE, ls, launch_fwd_uvu(a, tangent, pi.l_in, pi.l_out, g->n_nodes, ntiles, ls));
    seen[pi.out_block] = 1;
  }
  ETPC_HIP(lanes.finish());
  return ETPC_OK;
}

// ---------------------------------------------------------------- backward pieces (uvw)
struct UvwBwdReq {
  const float* x;         // features for Xt and W_bar (x^T P)
  const float* w;         // weights for Xt and x_bar (W^T P)
  const float* x2;        // second feature operand for W_bar with the plain state (x_dot^T P), or null
  const float* w2;        // second weight operand for x_bar with the plain state (w_dot^T P), or null
  const float* pos_dot;   // tangent direction (dbl) or null
  float* x_out;           // x_bar / x_grad or null
  float* w_out;           // W_bar / w_grad or null
  float* rbar;            // edge adjoint (first-order pass) or null
  bool tangent;           // dbl: the main state is the tangent state dP
  bool plain_needed;      // dbl: plain P needed for the x2 / w2 terms
  bool hess;              // dbl: rbar receives the position-Hessian term along pos_dot
  bool rbar_acc;          // add into rbar from the first path on (earlier passes wrote it)
  int lanes;              // concurrent lanes = edge-adjoint copies in use (rbar_lanes)
};

void wprep_args(const etpc_plan_s* p, const Derived& d, int k, const float* w, float* wcat, float* wt, WPrepArgs& a) {
  std::memset(&a, 0, sizeof(a));
  a.w = w;
  a.wcat = wcat;
  a.wt = wt;
  a.n_paths = static_cast<int32_t>(p->by_in[k].size());
  a.nb = p->n_basis;
  a.c_in = p->in[k].mul;
  a.ncols = static_cast<int32_t>(d.block_ncols[k]);
  for (int t = 0; t < a.n_paths; ++t) {
    const PathInfo& pi = p->paths[p->by_in[k][t]];
    a.path_off[t] = pi.w_off;
    a.col0[t] = d.block_col0[k][t];
    a.cout[t] = pi.c_out;
  }
}

// W_bar split-K partials of an item: wpart[split] = x^T state over the item's sender rows,
// for the item's ncols state columns; at most max_floats of partials (fewer splits if
// needed, at least one)
hipError_t wbar_gemm(const etpc_plan_s* p, int k, const float* xa, int64_t j0, int nsend, const float* state,
                     int64_t ncols, float* wpart, int64_t max_floats, int* splits_out, hipStream_t s) {
  const int ni = 2 * p->in[k].l + 1;
  const int c_in = p->in[k].mul;
  const int64_t K = static_cast<int64_t>(nsend) * ni;
  // enough splits for about kGemmTargetWg workgroups, at least 256 rows of K each (not
  // capped at kMaxSplits: an item of one path has few output tiles), within the partials' room
  const int64_t tiles = ((c_in + 63) / 64) * ((ncols + 63) / 64);
  int sp = static_cast<int>(
      std::max<int64_t>(1, std::min<int64_t>((kGemmTargetWg + tiles - 1) / tiles, (K + 255) / 256)));
  const int64_t per = static_cast<int64_t>(c_in) * ncols;
  sp = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(sp, max_floats / per)));
  int64_t ks = (K + sp - 1) / sp;
  ks = (ks + kGemmBK - 1) / kGemmBK * kGemmBK;
  sp = static_cast<int>((K + ks - 1) / ks);
  GemmArgs ga{};
  ga.lowp = p->gemm_precision;
  ga.A = xa + j0 * p->x_dim + p->xoff[k];
  ga.amap = irmul(ni, p->x_dim, c_in);
  ga.a_mcontig = 1;
  ga.B = state;
  ga.ldb = ncols;
  ga.C = wpart;
  ga.cmap = plain(ncols);
  ga.beta = 0;
  ga.M = c_in;
  ga.N = static_cast<int32_t>(ncols);
  ga.K = static_cast<int32_t>(K);
  ga.k_split = static_cast<int32_t>(ks);
  ga.c_split_stride = per;
  set_vec4(ga);
  *splits_out = sp;
  return launch_gemm(ga, sp, s);
}

// x_bar rows of an item (+)= state W^T over its ncols state columns (wt: the item's first
// row of the block's transposed weights)
etpc_status xbar_gemm(const etpc_plan_s* p, int k, const float* state, int64_t ncols, const float* wt, float* xo,
                      int64_t j0, int nsend, bool beta, const BwdLayout& L, hipStream_t s) {
  const int ni = 2 * p->in[k].l + 1;
  const int c_in = p->in[k].mul;
  GemmArgs ga{};
  ga.lowp = p->gemm_precision;
  ga.A = state;
  ga.amap = plain(ncols);
  ga.a_mcontig = 0;
  ga.B = wt;
  ga.ldb = c_in;
  ga.C = xo + j0 * p->x_dim + p->xoff[k];
  ga.cmap = irmul(ni, p->x_dim, c_in);
  ga.beta = beta ? 1 : 0;
  ga.M = nsend * ni;
  ga.N = c_in;
  ga.K = static_cast<int32_t>(ncols);
  return gemm_auto(ga, L.xpart, L.xpart_cap, kGemmSplits, ETPC_KIND_NODE_GEMM, s);
}

etpc_status bwd_uvw_run(const etpc_plan_s* p, const Derived& d, const etpc_graph* g, const float* pos,
                        const float* z_bar, const UvwBwdReq& R, const BwdLayout& L, const Sched& sch, hipStream_t s) {
  const GeomParams geom = p->geom();
  const int32_t N = g->n_nodes;
  const bool want_pos = R.rbar != nullptr;
  const bool main_state = R.tangent || (R.x_out || R.w_out);        // P (plain) or dP (tangent)
  const bool need_plain = R.tangent ? R.plain_needed : main_state;   // plain P
  const int nl = std::max(1, R.lanes);
  const int64_t rbar_stride = 3 * g->n_edges;
  if (R.x_out) ETPC_LAUNCH(ETPC_KIND_AUX, zero_unreached_in(p, R.x_out, N, s));
  // With two buffer sets, a software pipeline over the work items: while item i's
  // traversals run on the caller's stream and its lanes, the post stream re-lays out the
  // weights and forms Xt = x W for item i + 1 in the other set, then runs item i's x_bar /
  // W_bar GEMMs once its traversals are done.  With one set the items run one after
  // another on the caller's stream.
  const bool pipelined = L.nsets > 1;
  PostStream post(s, nl > 1 && pipelined);
  ETPC_HIP(post.status());
  const std::vector<Item> items = make_items(p, d, false, N, L.cap, sch.bounded);
  // weight re-layouts and Xt of one item into buffer set `b`, on stream `st`; with
  // `per_path`, one Xt GEMM per path of the item, each marked as a part of the post
  // work (st is then the post stream)
  auto prep = [&](const Item& it, int b, hipStream_t st, bool per_path) -> etpc_status {
    const int k = it.blk;
    const int ni = 2 * p->in[k].l + 1;
    const int c_in = p->in[k].mul;
    WPrepArgs wa;
    if (want_pos || R.x_out) {
      wprep_args(p, d, k, R.w, want_pos ? L.wcat[b] : nullptr, R.x_out ? L.wt[b] : nullptr, wa);
      ETPC_LAUNCH_ON(ETPC_KIND_AUX, st, launch_wprep(wa, st));
    }
    if (R.x_out && R.w2) {
      wprep_args(p, d, k, R.w2, nullptr, L.wt2[b], wa);
      ETPC_LAUNCH_ON(ETPC_KIND_AUX, st, launch_wprep(wa, st));
    }
    if (want_pos) {  // Xt = x W over the item's state columns
      GemmArgs ga{};
      ga.lowp = p->gemm_precision;
      ga.A = R.x + it.n0 * p->x_dim + p->xoff[k];
      ga.amap = irmul(ni, p->x_dim, c_in);
      ga.a_mcontig = 0;
      ga.B = L.wcat[b] + it.col0;
      ga.ldb = d.block_ncols[k];
      ga.C = L.xt[b];
      ga.cmap = plain(it.ncols);
      ga.beta = 0;
      ga.M = it.nn * ni;
      ga.N = static_cast<int32_t>(it.ncols);
      ga.K = c_in;
      ga.k_split = c_in;
      if (!per_path) {
        set_vec4(ga);
        ETPC_LAUNCH_ON(ETPC_KIND_NODE_GEMM, st, launch_gemm(ga, 1, st));
      } else {
        for (int t = it.t0; t < it.t1; ++t) {
          const int64_t c0 = d.block_col0[k][t] - it.col0;
          GemmArgs gp = ga;
          gp.B = ga.B + c0;
          gp.C = ga.C + c0;
          gp.N = static_cast<int32_t>(p->n_basis) * p->paths[p->by_in[k][t]].c_out;
          set_vec4(gp);
          ETPC_LAUNCH_ON(ETPC_KIND_NODE_GEMM, st, launch_gemm(gp, 1, st));
          ETPC_HIP(post.mark_part(t - it.t0));
        }
      }
    }
    return ETPC_OK;
  };
  // The first item's Xt has no earlier traversals to hide behind: with a post stream it
  // is formed there one path at a time, and each path's traversal waits only for its own
  // columns, so the traversals start after the first path's GEMM instead of the whole
  // item's.
  const bool split_first = pipelined && post.enabled() && want_pos && !items.empty() &&
                           items[0].t1 - items[0].t0 <= PostStream::kPostParts;
  if (pipelined && !items.empty()) {
    if (split_first) ETPC_HIP(post.follow());
    etpc_status st0 = split_first ? prep(items[0], 0, post.stream(), true) : prep(items[0], 0, s, false);
    if (st0 != ETPC_OK) return st0;
  }
  // Each lane's copy of the edge adjoint is first written by its first path (every item of
  // the fast schedule covers all senders).  Items of a bounded schedule may cover a sender
  // range several times, so there every copy starts at zero and every path accumulates.
  bool rbar_started[kLanes];
  for (int l = 0; l < kLanes; ++l) rbar_started[l] = R.rbar_acc || sch.bounded;
  if (want_pos && sch.bounded && !R.rbar_acc)
    ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(R.rbar, rbar_stride * nl, 0.f, s));
  // With the post stream the lanes stay forked for the whole pass: a lane goes on to the
  // next item's paths as soon as its own are done, after waiting for that item's Xt and
  // for the post work that last read the P set it writes; the post stream waits for every
  // lane before it reads P or overwrites an Xt set.
  const bool keep = post.enabled() && !capturing(s) && !sch.bounded;   // as in the forward
  std::optional<LaneGroup> pass_lanes;
  if (keep) {
    pass_lanes.emplace(s, nl);
    ETPC_HIP(pass_lanes->status());
  }
  int t_glob = 0;
  for (size_t ii = 0; ii < items.size(); ++ii) {
    const Item& it = items[ii];
    const int k = it.blk;
    const int set = pipelined ? static_cast<int>(ii & 1) : 0;
    const int nsend = it.nn;
    const auto& paths = p->by_in[k];
    const int c_in = p->in[k].mul;
    if (!pipelined) {
      etpc_status stp = prep(it, 0, s, false);
      if (stp != ETPC_OK) return stp;
    }
    // the next item's weights and Xt go into the other set, behind the post work of the
    // item that last used it
    if (pipelined && ii + 1 < items.size()) {
      // the previous item's traversals (which read that set's Xt) are enqueued before
      // this point: the post stream waits for them first
      if (keep) ETPC_HIP(pass_lanes->signal(post.stream()));
      ETPC_HIP(post.follow());
      etpc_status stp = prep(items[ii + 1], set ^ 1, post.stream(), false);
      if (stp != ETPC_OK) return stp;
      ETPC_HIP(post.ready(set ^ 1));
    }
    if (!keep) {
      ETPC_HIP(post.wait_ready(set));   // this item's Xt (prefetched, or made above on s)
      ETPC_HIP(post.wait_slot(set));    // its P set is no longer read by older post work
    }
    float* const Pset = L.P[set];
    float* const Pmain = R.tangent ? L.Pd[set] : L.P[set];
    // the item's paths write disjoint P columns and their own lane's edge adjoint copy
    std::optional<LaneGroup> item_lanes;
    if (!keep) {
      item_lanes.emplace(s, nl);
      ETPC_HIP(item_lanes->status());
    }
    LaneGroup& lanes = keep ? *pass_lanes : *item_lanes;
    unsigned waited = 0;   // kept lanes that already wait for this item's Xt and P sets
    for (int t = it.t0; t < it.t1; ++t, ++t_glob) {
      const PathInfo& pi = p->paths[paths[t]];
      const int lane = t_glob % nl;
      BwdUvwArgs a{};
      a.s_rowptr = g->s_rowptr;
      a.s_col = g->s_col;
      a.s_slot = g->s_slot;
      a.pos = pos;
      a.pos_dot = R.pos_dot;
      a.z_bar = z_bar;
      a.xt = L.xt[set];
      a.P = Pset;
      a.Pdot = L.Pd[set];
      a.rbar = R.rbar ? R.rbar + lane * rbar_stride : nullptr;
      a.send0 = static_cast<int32_t>(it.n0);
      a.order = (g->s_order != nullptr && it.n0 == 0 && nsend == g->n_nodes) ? g->s_order : nullptr;
      a.z_dim = static_cast<int32_t>(p->z_dim);
      a.zoff = static_cast<int32_t>(p->zoff[pi.out_block]);
      int ntiles = 1;
      a.cp = lane_width(pi.c_out, &ntiles, 16);
      a.c_out = pi.c_out;
      a.nparts = edge_parts(nsend, ntiles, g, pi.l_in, p->n_basis,
                            (R.hess ? 0 : (R.tangent ? need_plain : main_state) ? 1 : 0) + (R.tangent ? 1 : 0));
      a.ls = pi.l_sh;
      a.ld_state = it.ncols;
      a.state_col0 = d.block_col0[k][t] - it.col0;
      a.rbar_accumulate = rbar_started[lane] ? 1 : 0;
      a.g = geom;
      a.cg = pi.cgf;
      const bool np = R.tangent ? need_plain : main_state;
      const hipStream_t ls = lanes.lane(lane);
      if (keep && !(waited & (1u << lane))) {
        ETPC_HIP(post.wait_ready_on(ls, set));
        ETPC_HIP(post.wait_slot_on(ls, set));
        waited |= 1u << lane;
      }
      if (split_first && ii == 0) ETPC_HIP(post.wait_part(ls, t - it.t0));
      ETPC_LAUNCH_ON(ETPC_KIND_BWD_TRAVERSE, ls,
                     launch_bwd_uvw(a, R.hess ? false : np, want_pos, R.tangent, R.hess, pi.l_in, pi.l_out, nsend,
                                    ntiles, ls));
      if (want_pos) rbar_started[lane] = true;
    }
    if (keep)
      ETPC_HIP(lanes.signal(post.stream()));
    else
      ETPC_HIP(lanes.finish());
    if (R.x_out || R.w_out) {
      ETPC_HIP(post.follow());
      const hipStream_t ps = post.stream();
      // The last item's products end the pass with nothing beside them: its x_bar GEMM runs
      // on the caller's stream (once every lane and the previous item's post work, which
      // used the same split-K partials, are done) beside its W_bar GEMM on the post stream
      // (workload 2 2.60 -> 2.58 ms, workload 5 3.29 -> 3.26 ms).
      hipStream_t xs = ps;
      if (keep && ii + 1 == items.size() && R.x_out && R.w_out) {
        ETPC_HIP(pass_lanes->signal(s));
        ETPC_HIP(post.wait_slot(set ^ 1));
        xs = s;
      }
      if (R.x_out) {
        // the first path subset of a sender range writes its x_bar rows, later ones add
        const float* wt_main = L.wt[set] + it.col0 * c_in;
        if (main_state) {
          etpc_status st = xbar_gemm(p, k, Pmain, it.ncols, wt_main, R.x_out, it.n0, nsend, it.t0 > 0, L, xs);
          if (st != ETPC_OK) return st;
        }
        if (R.tangent && R.w2) {
          etpc_status st = xbar_gemm(p, k, Pset, it.ncols, L.wt2[set] + it.col0 * c_in, R.x_out, it.n0, nsend, true,
                                     L, xs);
          if (st != ETPC_OK) return st;
        }
      }
      if (R.w_out) {
        int sp1 = 0, sp2 = 0;
        const bool two = R.tangent && R.x2;
        const int64_t room = two ? L.wpart_cap / 2 : L.wpart_cap;
        ETPC_LAUNCH_ON(ETPC_KIND_NODE_GEMM, ps,
                       wbar_gemm(p, k, R.x, it.n0, nsend, Pmain, it.ncols, L.wpart, room, &sp1, ps));
        if (two)
          ETPC_LAUNCH_ON(ETPC_KIND_NODE_GEMM, ps,
                         wbar_gemm(p, k, R.x2, it.n0, nsend, Pset, it.ncols,
                                   L.wpart + static_cast<int64_t>(sp1) * c_in * it.ncols, room, &sp2, ps));
        int64_t poff[kMaxPaths];
        int32_t col0[kMaxPaths], cout[kMaxPaths];
        const int npath = it.t1 - it.t0;
        for (int t = 0; t < npath; ++t) {
          poff[t] = p->paths[paths[it.t0 + t]].w_off;
          col0[t] = static_cast<int32_t>(d.block_col0[k][it.t0 + t] - it.col0);
          cout[t] = p->paths[paths[it.t0 + t]].c_out;
        }
        // the first sender range of a path writes its W_bar block, later ones add
        ETPC_LAUNCH_ON(ETPC_KIND_AUX, ps,
                       launch_reduce_wbar(L.wpart, sp1 + sp2, c_in, npath, p->n_basis, poff, col0, cout,
                                          static_cast<int>(it.ncols), R.w_out, it.n0 > 0, ps));
      }
      ETPC_HIP(post.mark(set));
    }
  }
  if (keep) ETPC_HIP(pass_lanes->finish());
  ETPC_HIP(post.finish());
  return ETPC_OK;
}

// ---------------------------------------------------------------- backward pieces (uvu)
struct UvuBwdReq {
  const float* x;
  const float* w;
  const float* pos_dot;
  float* x_out;
  float* w_out;
  float* rbar;
  bool tangent;
  bool x_acc;     // accumulate into x_out from the first path on
  bool w_acc;     // accumulate into w_out
  bool hess;      // rbar receives the position-Hessian term along pos_dot (no x_out / w_out)
  bool rbar_acc;  // add into rbar from the first path on
  int lanes;      // concurrent lanes = edge-adjoint and W_bar partial copies in use
};

etpc_status bwd_uvu_run(const etpc_plan_s* p, const etpc_graph* g, const float* pos, const float* z_bar,
                        const UvuBwdReq& R, const BwdLayout& L, hipStream_t s) {
  const GeomParams geom = p->geom();
  const int32_t N = g->n_nodes;
  const int grid = static_cast<int>(std::min<int64_t>(N, kUvuGrid));
  if (R.x_out && !R.x_acc) ETPC_LAUNCH(ETPC_KIND_AUX, zero_unreached_in(p, R.x_out, N, s));
  std::vector<int> seen(p->in.size(), 0);
  // one lane per input block (x_bar accumulates per block); per-lane edge adjoint and
  // W_bar partial copies
  const int nl = std::max(1, R.lanes);
  const std::vector<int> lane_of = block_lanes(p, true, nl);
  const int64_t rbar_stride = 3 * g->n_edges;
  bool rbar_started[kLanes];
  for (int l = 0; l < kLanes; ++l) rbar_started[l] = R.rbar_acc;
  LaneGroup lanes(s, nl);
  ETPC_HIP(lanes.status());
  for (const PathInfo& pi : p->paths) {
    const int lane = lane_of[pi.in_block];
    float* wpart = R.w_out ? L.wpart + lane * L.wpart_lane : nullptr;
    BwdUvuArgs a{};
    a.s_rowptr = g->s_rowptr;
    a.s_col = g->s_col;
    a.s_slot = g->s_slot;
    a.pos = pos;
    a.pos_dot = R.pos_dot;
    a.x = R.x;
    a.w = R.w + pi.w_off;
    a.z_bar = z_bar;
    a.x_bar = R.x_out;
    a.wbar_part = wpart;
    a.rbar = R.rbar ? R.rbar + lane * rbar_stride : nullptr;
    a.n_nodes = N;
    a.x_dim = static_cast<int32_t>(p->x_dim);
    a.xoff = static_cast<int32_t>(p->xoff[pi.in_block]);
    a.z_dim = static_cast<int32_t>(p->z_dim);
    a.zoff = static_cast<int32_t>(p->zoff[pi.out_block]);
    int ntiles = 1;
    a.cp = lane_width(pi.c_in, &ntiles, 16);
    a.c = pi.c_in;
    a.ls = pi.l_sh;
    a.xbar_accumulate = (R.x_acc || seen[pi.in_block]) ? 1 : 0;
    a.rbar_accumulate = rbar_started[lane] ? 1 : 0;
    a.g = geom;
    a.cg = pi.cgf;
    const hipStream_t ls = lanes.lane(lane);
    ETPC_LAUNCH_ON(ETPC_KIND_BWD_TRAVERSE, ls,
                   launch_bwd_uvu(a, R.tangent, R.hess, pi.l_in, pi.l_out, grid, ntiles, ls));
    seen[pi.in_block] = 1;
    if (R.rbar) rbar_started[lane] = true;
    if (R.w_out) {
      int64_t poff[1] = {pi.w_off};
      int32_t col0[1] = {0}, cout[1] = {pi.c_in};
      ETPC_LAUNCH_ON(ETPC_KIND_AUX, ls,
                     launch_reduce_wbar(wpart, grid, 1, 1, p->n_basis, poff, col0, cout, p->n_basis * pi.c_in,
                                        R.w_out, R.w_acc, ls));
    }
  }
  ETPC_HIP(lanes.finish());
  return ETPC_OK;
}

// Forward on a caller-given workspace (uvw: node chunks that fit; uvu needs none).
etpc_status forward_impl(const etpc_plan_s* p, const etpc_graph* g, const float* x, const float* pos, const float* w,
                         float* z, void* ws, size_t ws_bytes, int nl, hipStream_t s) {
  const Derived d = derive(p);
  const int64_t N = g->n_nodes;
  auto bytes_of = [&](int64_t c, const Sched& sc) { return fwd_bytes(p, d, N, c, sc); };
  Sched sch;
  int64_t cap = 0;
  choose_schedule(p, d, true, false, N, g->n_edges, ws_bytes, bytes_of, &sch, &cap);
  if (p->mode == ETPC_UVW) {
    etpc_status st = check_ws(ws, ws_bytes, bytes_of(cap < 0 ? min_cap(p, true, false) : cap, sch));
    if (st != ETPC_OK) return st;
  }
  Carver c{static_cast<char*>(ws), 0};
  FwdLayout L;
  fwd_layout(p, d, N, std::max<int64_t>(cap, 0), sch, c, L);
  ETPC_LAUNCH(ETPC_KIND_AUX, zero_unreached(p, z, g->n_nodes, s));
  if (p->mode == ETPC_UVW) return fwd_uvw_run(p, d, g, x, pos, nullptr, w, z, false, false, L, sch, nl, s);
  return fwd_uvu_run(p, g, x, pos, nullptr, w, z, false, false, nl, s);
}

// ---------------------------------------------------------------- fixed scratch
// Device scratch of etpc_forward_noalloc, for callers that cannot allocate: a file-scope
// device array (one copy per GPU, resident until the process ends), 128 MiB, the
// tensor-product scratch cap the Sobek paper's measurements use (Sec. 5).  In host code
// the array's name only stands in for the symbol: its device address (one per device) is
// taken once per device with hipGetSymbolAddress and only that address is passed on.
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's address of `scratch`, looked up on the first call on that device.
etpc_status static_scratch(void** out) {
  int dev = 0;
  ETPC_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices) ETPC_FAIL(ETPC_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    ETPC_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (ptr == nullptr) ETPC_FAIL(ETPC_ERR_HIP, "hipGetSymbolAddress returned no address for the fixed scratch");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ETPC_OK;
}

}  // namespace

extern "C" {

etpc_status etpc_workspace_size(etpc_plan p, int32_t pass, int32_t n_nodes, int64_t n_edges, size_t budget,
                                size_t* bytes) {
  if (p == nullptr || bytes == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null plan or output");
  if (n_nodes < 0 || n_edges < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative graph size");
  if (pass != ETPC_PASS_FWD && pass != ETPC_PASS_BWD && pass != ETPC_PASS_DBL)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "unknown pass");
  const Derived d = derive(p);
  const bool fwd = pass != ETPC_PASS_BWD, bwd = pass != ETPC_PASS_FWD;
  // uvu keeps no node state: its layout depends on the persistent grid, not on a buffer size
  auto bytes_of = [&](int64_t c, const Sched& sc) -> size_t {
    if (pass == ETPC_PASS_FWD) return fwd_bytes(p, d, n_nodes, c, sc);
    if (pass == ETPC_PASS_BWD) return bwd_bytes(p, d, n_nodes, n_edges, c, sc);
    return dbl_bytes(p, d, n_nodes, n_edges, c, sc);
  };
  const size_t full = bytes_of(p->mode == ETPC_UVW ? full_cap(d, n_nodes, fwd, bwd) : 0, fast_sched(p, n_edges));
  if (budget == 0 || full <= budget || n_nodes == 0) {
    *bytes = full;
    return ETPC_OK;
  }
  Sched sch;
  int64_t cap = 0;
  choose_schedule(p, d, fwd, bwd, n_nodes, n_edges, budget, bytes_of, &sch, &cap);
  if (cap < 0) {
    *bytes = bytes_of(min_cap(p, fwd, bwd), sch);
    ETPC_FAIL(ETPC_ERR_WORKSPACE, "budget below the pass's minimum of " + std::to_string(*bytes) + " bytes");
  }
  *bytes = bytes_of(cap, sch);
  return ETPC_OK;
}

etpc_status etpc_csr_workspace_size(int32_t n_nodes, int64_t n_edges, size_t* bytes) {
  if (bytes == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null output");
  if (n_nodes < 0 || n_edges < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative graph size");
  *bytes = csr_workspace_bytes(n_nodes, n_edges);
  return ETPC_OK;
}

etpc_status etpc_csr_build(int32_t n_nodes, int64_t n_edges, const int32_t* src, const int32_t* dst, int32_t* rowptr,
                           int32_t* col, int32_t* eid, int32_t* s_rowptr, int32_t* s_col, int32_t* s_slot, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (n_nodes < 0 || n_edges < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative graph size");
  if (n_edges >= (int64_t(1) << 31)) ETPC_FAIL(ETPC_ERR_OVERFLOW, "n_edges must be < 2^31");
  if (rowptr == nullptr || s_rowptr == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null row pointer outputs");
  if (n_edges > 0 && (src == nullptr || dst == nullptr || col == nullptr || eid == nullptr || s_col == nullptr ||
                      s_slot == nullptr))
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null edge arrays");
  if (n_edges > 0 && n_nodes == 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "edges on an empty node set");
  etpc_status st = check_ws(ws, ws_bytes, csr_workspace_bytes(n_nodes, n_edges));
  if (st != ETPC_OK) return st;
  ::etpc::ProfScope ps(ETPC_KIND_CSR, stream);
  return csr_build_impl(n_nodes, n_edges, src, dst, rowptr, col, eid, s_rowptr, s_col, s_slot, ws, stream);
}

etpc_status etpc_degree_order_workspace_size(int32_t n_nodes, size_t* bytes) {
  if (bytes == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null output");
  if (n_nodes < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative node count");
  *bytes = degree_order_bytes(n_nodes);
  return ETPC_OK;
}

etpc_status etpc_degree_order(int32_t n_nodes, const int32_t* rowptr, int32_t window, int32_t* order, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (n_nodes < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative node count");
  if (window < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative window");
  if (n_nodes == 0) return ETPC_OK;
  if (rowptr == nullptr || order == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null arrays");
  etpc_status st = check_ws(ws, ws_bytes, degree_order_bytes(n_nodes));
  if (st != ETPC_OK) return st;
  ::etpc::ProfScope ps(ETPC_KIND_CSR, stream);
  return degree_order_impl(n_nodes, rowptr, window, nullptr, order, ws, stream);
}

etpc_status etpc_degree_order_within(int32_t n_nodes, const int32_t* rowptr, int32_t window, const int32_t* base,
                                     int32_t* order, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_nodes < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative node count");
  if (window < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative window");
  if (n_nodes == 0) return ETPC_OK;
  if (rowptr == nullptr || base == nullptr || order == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null arrays");
  etpc_status st = check_ws(ws, ws_bytes, degree_order_bytes(n_nodes));
  if (st != ETPC_OK) return st;
  ::etpc::ProfScope ps(ETPC_KIND_CSR, stream);
  return degree_order_impl(n_nodes, rowptr, window, base, order, ws, stream);
}

etpc_status etpc_spatial_order_workspace_size(int32_t n_nodes, size_t* bytes) {
  if (bytes == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null output");
  if (n_nodes < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative node count");
  *bytes = spatial_order_bytes(n_nodes);
  return ETPC_OK;
}

etpc_status etpc_spatial_order(int32_t n_nodes, const float* pos, const float* box, int32_t* order, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  if (n_nodes < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative node count");
  if (n_nodes == 0) return ETPC_OK;
  if (pos == nullptr || order == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null arrays");
  if (box != nullptr)
    for (int d = 0; d < 3; ++d)
      if (!(box[d] > 0.f) || !std::isfinite(box[d])) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "box lengths must be finite and > 0");
  etpc_status st = check_ws(ws, ws_bytes, spatial_order_bytes(n_nodes));
  if (st != ETPC_OK) return st;
  ::etpc::ProfScope ps(ETPC_KIND_CSR, stream);
  return spatial_order_impl(n_nodes, pos, box, order, ws, stream);
}

etpc_status etpc_graph_validate(const etpc_graph* g, hipStream_t stream) {
  if (g == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null graph");
  if (g->n_nodes < 0 || g->n_edges < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative graph size");
  if (g->n_edges >= (int64_t(1) << 31)) ETPC_FAIL(ETPC_ERR_OVERFLOW, "n_edges must be < 2^31");
  if (g->rowptr == nullptr || g->s_rowptr == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null row pointers");
  if (g->n_edges > 0 && (g->col == nullptr || g->s_col == nullptr || g->s_slot == nullptr))
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null CSR index arrays");
  return graph_validate_impl(*g, stream);
}

etpc_status etpc_radius_graph_workspace_size(int32_t n_nodes, int64_t max_edges, size_t* bytes) {
  if (bytes == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null output");
  if (n_nodes < 0 || max_edges < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative size");
  if (n_nodes >= (1 << 30)) ETPC_FAIL(ETPC_ERR_OVERFLOW, "n_nodes must be < 2^30");
  *bytes = radius_workspace_bytes(n_nodes, max_edges);
  return ETPC_OK;
}

etpc_status etpc_radius_graph(int32_t n_nodes, const float* pos, float cutoff, const float* box, int64_t max_edges,
                              int32_t* src, int32_t* dst, int64_t* n_edges, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (n_edges == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null n_edges");
  *n_edges = 0;
  if (n_nodes < 0 || max_edges < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative size");
  if (n_nodes >= (1 << 30)) ETPC_FAIL(ETPC_ERR_OVERFLOW, "n_nodes must be < 2^30");
  if (!(cutoff > 0.f) || !std::isfinite(cutoff)) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "cutoff must be positive and finite");
  if (box != nullptr)
    for (int a = 0; a < 3; ++a) {
      if (!(box[a] > 0.f) || !std::isfinite(box[a])) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "box lengths must be positive");
      if (box[a] < 2.f * cutoff)
        ETPC_FAIL(ETPC_ERR_INVALID_ARG, "cutoff exceeds half the box: the minimum image is not unique");
    }
  if (n_nodes == 0) return ETPC_OK;
  if (pos == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null positions");
  if (max_edges > 0 && (src == nullptr || dst == nullptr)) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null edge outputs");
  etpc_status st = check_ws(ws, ws_bytes, radius_workspace_bytes(n_nodes, max_edges));
  if (st != ETPC_OK) return st;
  return radius_graph_impl(n_nodes, pos, cutoff, box, max_edges, src, dst, n_edges, ws, stream);
}

etpc_status etpc_layout_convert(etpc_plan p, int32_t features, int32_t direction, int32_t n_nodes, const float* in,
                                float* out, hipStream_t stream) {
  if (p == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null plan");
  if (features != ETPC_FEATURES_IN && features != ETPC_FEATURES_OUT) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "bad features");
  if (direction != ETPC_TO_IR_MUL && direction != ETPC_TO_MUL_IR) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "bad direction");
  if (n_nodes < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "negative n_nodes");
  if (n_nodes == 0) return ETPC_OK;
  if (in == nullptr || out == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null in or out");
  const std::vector<etpc_irrep>& ir = features == ETPC_FEATURES_IN ? p->in : p->out;
  const int64_t width = features == ETPC_FEATURES_IN ? p->x_dim : p->z_dim;
  if (static_cast<int64_t>(n_nodes) * width >= (int64_t(1) << 40)) ETPC_FAIL(ETPC_ERR_OVERFLOW, "too many elements");
  const char* a = reinterpret_cast<const char*>(in);
  const char* b = reinterpret_cast<const char*>(out);
  const size_t bytes = static_cast<size_t>(n_nodes) * static_cast<size_t>(width) * sizeof(float);
  if (a < b + bytes && b < a + bytes) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "in and out overlap");
  return layout_convert_impl(ir, direction, n_nodes, in, out, stream);
}

etpc_status etpc_forward(etpc_plan p, const etpc_graph* g, const float* x, const float* pos, const float* w, float* z,
                         void* ws, size_t ws_bytes, hipStream_t s) {
  etpc_status st = check_common(p, g);
  if (st != ETPC_OK) return st;
  if (g->n_nodes == 0) return ETPC_OK;
  if (x == nullptr || pos == nullptr || w == nullptr || z == nullptr)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null x, pos, w or z");
  return forward_impl(p, g, x, pos, w, z, ws, ws_bytes, lane_cap(p, g), s);
}

etpc_status etpc_forward_noalloc(etpc_plan p, const etpc_graph* g, const float* x, const float* pos, const float* w,
                                 float* z, hipStream_t s) {
  etpc_status st = check_common(p, g);
  if (st != ETPC_OK) return st;
  if (g->n_nodes == 0) return ETPC_OK;
  if (x == nullptr || pos == nullptr || w == nullptr || z == nullptr)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null x, pos, w or z");
  if (p->mode == ETPC_UVU) return forward_impl(p, g, x, pos, w, z, nullptr, 0, 1, s);   // no scratch
  const Derived d = derive(p);
  Sched one_set;
  one_set.bounded = true;
  one_set.nsets = 1;
  const size_t one = fwd_bytes(p, d, g->n_nodes, min_cap(p, true, false), one_set);
  if (one > kStaticScratchBytes)
    ETPC_FAIL(ETPC_ERR_WORKSPACE, "one receiver's state (" + std::to_string(one) +
                                      " bytes) exceeds the fixed scratch of " +
                                      std::to_string(kStaticScratchBytes) + " bytes");
  void* ptr = nullptr;
  st = static_scratch(&ptr);
  if (st != ETPC_OK) return st;
  // one lane: the side streams would be created on first use, which this entry point avoids
  return forward_impl(p, g, x, pos, w, z, ptr, kStaticScratchBytes, 1, s);
}

etpc_status etpc_backward(etpc_plan p, const etpc_graph* g, const float* x, const float* pos, const float* w,
                          const float* z_bar, float* x_bar, float* w_bar, float* pos_bar, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  etpc_status st = check_common(p, g);
  if (st != ETPC_OK) return st;
  if (x == nullptr || pos == nullptr || w == nullptr || z_bar == nullptr)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null x, pos, w or z_bar");
  st = check_channels_bwd(p);
  if (st != ETPC_OK) return st;
  if (x_bar == nullptr && w_bar == nullptr && pos_bar == nullptr) return ETPC_OK;
  const Derived d = derive(p);
  const bool want_pos = pos_bar != nullptr;
  const bool need_p = x_bar || w_bar;
  const int32_t N = g->n_nodes;
  if (N == 0) {
    if (w_bar) ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(w_bar, p->w_numel, 0.f, s));
    return ETPC_OK;
  }
  auto bytes_of = [&](int64_t c, const Sched& sc) {
    Carver cv;
    BwdLayout L;
    bwd_layout(p, d, N, g->n_edges, p->mode == ETPC_UVW ? c : kUvuGrid, sc, want_pos, need_p, false,
               w_bar != nullptr, false, x_bar != nullptr, false, cv, L);
    return cv.off;
  };
  Sched sch;
  int64_t cap = 0;
  choose_schedule(p, d, false, true, N, g->n_edges, ws_bytes, bytes_of, &sch, &cap);
  st = check_ws(ws, ws_bytes, bytes_of(cap < 0 ? min_cap(p, false, true) : cap, sch));
  if (st != ETPC_OK) return st;
  // concurrent lanes = edge-adjoint copies the schedule keeps
  const int lanes = want_pos ? std::min(rbar_lanes(p, g), sch.rbar_copies) : rbar_lanes(p, g);
  Carver cv{static_cast<char*>(ws), 0};
  BwdLayout L;
  bwd_layout(p, d, N, g->n_edges, p->mode == ETPC_UVW ? cap : kUvuGrid, sch, want_pos, need_p, false,
             w_bar != nullptr, false, x_bar != nullptr, false, cv, L);
  if (p->mode == ETPC_UVW) {
    UvwBwdReq R{};
    R.lanes = lanes;
    R.x = x;
    R.w = w;
    R.x_out = x_bar;
    R.w_out = w_bar;
    R.rbar = want_pos ? L.rbar : nullptr;
    st = bwd_uvw_run(p, d, g, pos, z_bar, R, L, sch, s);
  } else {
    UvuBwdReq R{};
    R.lanes = lanes;
    R.x = x;
    R.w = w;
    R.x_out = x_bar;
    R.w_out = w_bar;
    R.rbar = want_pos ? L.rbar : nullptr;
    st = bwd_uvu_run(p, g, pos, z_bar, R, L, s);
  }
  if (st != ETPC_OK) return st;
  if (want_pos) {
    if (g->n_edges == 0 || p->paths.empty()) {
      ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(pos_bar, 3 * static_cast<int64_t>(N), 0.f, s));
    } else {
      ETPC_LAUNCH(ETPC_KIND_AUX, launch_pos_bar(g->rowptr, g->s_rowptr, g->s_slot, L.rbar, lanes,
                                                g->n_edges, pos_bar, N, s));
    }
  }
  if (w_bar && p->paths.empty()) ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(w_bar, p->w_numel, 0.f, s));
  return ETPC_OK;
}

etpc_status etpc_double_backward(etpc_plan p, const etpc_graph* g, const float* x, const float* pos, const float* w,
                                 const float* z_bar, const float* x_dot, const float* w_dot, const float* pos_dot,
                                 float* z_bar_grad, float* x_grad, float* w_grad, float* pos_grad, void* ws,
                                 size_t ws_bytes, hipStream_t s) {
  etpc_status st = check_common(p, g);
  if (st != ETPC_OK) return st;
  if (x == nullptr || pos == nullptr || w == nullptr || z_bar == nullptr)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null x, pos, w or z_bar");
  st = check_channels_bwd(p);
  if (st != ETPC_OK) return st;
  const int32_t N = g->n_nodes;
  if (N == 0) {
    if (w_grad) ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(w_grad, p->w_numel, 0.f, s));
    return ETPC_OK;
  }
  const bool want_pos = pos_grad != nullptr;
  const Derived d = derive(p);
  const bool tan = pos_dot != nullptr;
  const bool plain = x_dot != nullptr || w_dot != nullptr;
  auto bytes_of = [&](int64_t c, const Sched& sc) {
    Carver cv;
    BwdLayout L;
    const int64_t ch = p->mode == ETPC_UVW ? c : kUvuGrid;
    bwd_layout(p, d, N, g->n_edges, ch, sc, want_pos, plain, tan, w_grad != nullptr, tan && x_dot, x_grad != nullptr,
               x_grad && w_dot && tan, cv, L);
    return std::max(cv.off, z_bar_grad ? fwd_bytes(p, d, N, c, sc) : size_t(0));
  };
  Sched sch;
  int64_t cap = 0;
  const bool fwd_state = z_bar_grad != nullptr;
  choose_schedule(p, d, fwd_state, true, N, g->n_edges, ws_bytes, bytes_of, &sch, &cap);
  st = check_ws(ws, ws_bytes, bytes_of(cap < 0 ? min_cap(p, fwd_state, true) : cap, sch));
  if (st != ETPC_OK) return st;
  const int64_t chunk = p->mode == ETPC_UVW ? cap : kUvuGrid;
  const int lanes = want_pos ? std::min(rbar_lanes(p, g), sch.rbar_copies) : rbar_lanes(p, g);

  // d/dz_bar = z_dot = J_pos pos_dot + J_x x_dot + J_W w_dot (forward tangents)
  if (z_bar_grad) {
    Carver cv{static_cast<char*>(ws), 0};
    FwdLayout L;
    fwd_layout(p, d, N, cap, sch, cv, L);
    if (!tan && !plain) {
      ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(z_bar_grad, static_cast<int64_t>(N) * p->z_dim, 0.f, s));
    } else {
      ETPC_LAUNCH(ETPC_KIND_AUX, zero_unreached(p, z_bar_grad, N, s));
      bool beta = false;
      for (int term = 0; term < 3; ++term) {
        const float* xin = x;
        const float* win = w;
        bool tangent = false;
        if (term == 0) {
          if (!tan) continue;
          tangent = true;
        } else if (term == 1) {
          if (!x_dot) continue;
          xin = x_dot;
        } else {
          if (!w_dot) continue;
          win = w_dot;
        }
        if (p->mode == ETPC_UVW)
          st = fwd_uvw_run(p, d, g, xin, pos, pos_dot, win, z_bar_grad, beta, tangent, L, sch, lane_cap(p, g), s);
        else
          st = fwd_uvu_run(p, g, xin, pos, pos_dot, win, z_bar_grad, beta, tangent, lane_cap(p, g), s);
        if (st != ETPC_OK) return st;
        beta = true;
      }
    }
  }
  // d/dx and d/dW
  auto xw_part = [&]() -> etpc_status {
    if (!x_grad && !w_grad) return ETPC_OK;
    if (!tan && !plain) {
      if (x_grad) ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(x_grad, static_cast<int64_t>(N) * p->x_dim, 0.f, s));
      if (w_grad) ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(w_grad, p->w_numel, 0.f, s));
      return ETPC_OK;
    }
    Carver cv{static_cast<char*>(ws), 0};
    BwdLayout L;
    const int64_t ch = p->mode == ETPC_UVW ? chunk : kUvuGrid;
    bwd_layout(p, d, N, g->n_edges, ch, sch, want_pos, plain, tan, w_grad != nullptr, tan && x_dot, x_grad != nullptr,
               x_grad && w_dot && tan, cv, L);
    if (p->mode == ETPC_UVW) {
      // d/dx = W^T dP + w_dot^T P ;  d/dW = x^T dP + x_dot^T P
      UvwBwdReq R{};
      R.lanes = lanes;
      R.pos_dot = pos_dot;
      if (tan) {
        R.x = x;
        R.w = w;
        R.x2 = x_dot;
        R.w2 = w_dot;
        R.tangent = true;
        R.plain_needed = plain;
      } else {
        // only plain terms: x_grad = w_dot^T P, w_grad = x_dot^T P (zero where the cotangent is absent)
        R.x = x_dot;
        R.w = w_dot;
        R.tangent = false;
      }
      R.x_out = x_grad;
      R.w_out = w_grad;
      if (!tan) {
        if (x_grad && !w_dot) {
          ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(x_grad, static_cast<int64_t>(N) * p->x_dim, 0.f, s));
          R.x_out = nullptr;
        }
        if (w_grad && !x_dot) {
          ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(w_grad, p->w_numel, 0.f, s));
          R.w_out = nullptr;
        }
        if (!R.x_out && !R.w_out) return ETPC_OK;
        // the plain pass reads x (for W_bar) and w (for x_bar); feed the cotangents in their place
        R.x = x_dot ? x_dot : x;
        R.w = w_dot ? w_dot : w;
      }
      return bwd_uvw_run(p, d, g, pos, z_bar, R, L, sch, s);
    }
    // uvu: tangent pass (pos_dot) then plain passes with w -> w_dot (x_grad) and x -> x_dot (w_grad)
    bool xs = false, wsd = false;
    if (tan) {
      UvuBwdReq R{};
      R.lanes = lanes;
      R.x = x;
      R.w = w;
      R.pos_dot = pos_dot;
      R.tangent = true;
      R.x_out = x_grad;
      R.w_out = w_grad;
      st = bwd_uvu_run(p, g, pos, z_bar, R, L, s);
      if (st != ETPC_OK) return st;
      xs = x_grad != nullptr;
      wsd = w_grad != nullptr;
    }
    if (x_grad && w_dot) {
      UvuBwdReq R{};
      R.lanes = lanes;
      R.x = x;
      R.w = w_dot;
      R.x_out = x_grad;
      R.x_acc = xs;
      st = bwd_uvu_run(p, g, pos, z_bar, R, L, s);
      if (st != ETPC_OK) return st;
      xs = true;
    }
    if (w_grad && x_dot) {
      UvuBwdReq R{};
      R.lanes = lanes;
      R.x = x_dot;
      R.w = w;
      R.w_out = w_grad;
      R.w_acc = wsd;
      st = bwd_uvu_run(p, g, pos, z_bar, R, L, s);
      if (st != ETPC_OK) return st;
      wsd = true;
    }
    if (x_grad && !xs) ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(x_grad, static_cast<int64_t>(N) * p->x_dim, 0.f, s));
    if (w_grad && !wsd) ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(w_grad, p->w_numel, 0.f, s));
  return ETPC_OK;
  };
  st = xw_part();
  if (st != ETPC_OK) return st;
  if (!want_pos) return ETPC_OK;

  // d/dpos: pos_bar of the backward with x -> x_dot and with W -> w_dot (the x_bar and
  // W_bar cotangents enter <z_bar, z> linearly), plus the edge Hessian H_e r_dot_e of
  // the pos_dot term; all three accumulate into the per-edge buffer, then one segment sum.
  if ((!tan && !plain) || g->n_edges == 0 || p->paths.empty()) {
    ETPC_LAUNCH(ETPC_KIND_AUX, launch_fill(pos_grad, 3 * static_cast<int64_t>(N), 0.f, s));
    return ETPC_OK;
  }
  Carver cvp{static_cast<char*>(ws), 0};
  BwdLayout Lp;
  const int64_t chp = p->mode == ETPC_UVW ? chunk : kUvuGrid;
  bwd_layout(p, d, N, g->n_edges, chp, sch, true, false, false, false, false, false, false, cvp, Lp);
  bool acc = false;
  for (int term = 0; term < 3; ++term) {
    const float* xin = x;
    const float* win = w;
    bool hess = false;
    if (term == 0) {
      if (!x_dot) continue;
      xin = x_dot;
    } else if (term == 1) {
      if (!w_dot) continue;
      win = w_dot;
    } else {
      if (!tan) continue;
      hess = true;
    }
    if (p->mode == ETPC_UVW) {
      UvwBwdReq R{};
      R.lanes = lanes;
      R.x = xin;
      R.w = win;
      R.pos_dot = hess ? pos_dot : nullptr;
      R.rbar = Lp.rbar;
      R.hess = hess;
      R.rbar_acc = acc;
      st = bwd_uvw_run(p, d, g, pos, z_bar, R, Lp, sch, s);
    } else {
      UvuBwdReq R{};
      R.lanes = lanes;
      R.x = xin;
      R.w = win;
      R.pos_dot = hess ? pos_dot : nullptr;
      R.rbar = Lp.rbar;
      R.hess = hess;
      R.rbar_acc = acc;
      st = bwd_uvu_run(p, g, pos, z_bar, R, Lp, s);
    }
    if (st != ETPC_OK) return st;
    acc = true;
  }
  ETPC_LAUNCH(ETPC_KIND_AUX, launch_pos_bar(g->rowptr, g->s_rowptr, g->s_slot, Lp.rbar, lanes, g->n_edges,
                                            pos_grad, N, s));
  return ETPC_OK;
}

}  // extern "C"
