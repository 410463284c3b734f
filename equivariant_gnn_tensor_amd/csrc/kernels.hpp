// Kernel argument blocks and launchers (internal).
#pragma once

#include "common.hpp"

namespace etpc {

// ---------------------------------------------------------------- forward, uvw
// One receiver traversal for one path: S[(i, m_out)][col0 + q*C_in + u]
//   = sum_{e -> i} phi_q(r_e) sum_{m_in} x_j[u, m_in] cY_e[m_in, m_out]
// (Sobek paper, Sec. 4, Eq. 32-33).  With `tangent`, accumulates the position
// tangent dS = sum_e (dphi_q C + phi_q dC) instead, for the direction pos_dot.
struct FwdUvwArgs {
  const int32_t* rowptr;
  const int32_t* col;
  const float* pos;
  const float* pos_dot;   // tangent only
  const float* x;
  float* S;
  const int32_t* order;   // node slot b takes receiver order[b] (whole-graph launches), or null
  int32_t recv0;          // first receiver of this chunk
  int32_t x_dim, xoff, c_in, cp;
  int32_t ls;
  int64_t s_row_stride;   // D_g (floats per S row)
  int32_t s_col0;         // column offset of this path inside the group
  int32_t nparts;         // waves that split a receiver's edges (1..4)
  GeomParams g;
  CGTable cg;
};
hipError_t launch_fwd_uvw(const FwdUvwArgs& a, bool tangent, int li, int lo, int nrecv, int ntiles, hipStream_t s);

// ---------------------------------------------------------------- forward, uvu
// z_i[g, u, m_out] (+)= sum_{e -> i} (sum_q phi_q W[q,u]) sum_{m_in} x_j[u,m_in] cY_e[m_in,m_out]
// (Eq. 7 with the edge-local weight of Eq. 17).
struct FwdUvuArgs {
  const int32_t* rowptr;
  const int32_t* col;
  const float* pos;
  const float* pos_dot;   // tangent only
  const float* x;
  const float* w;         // path block [B][C]
  float* z;
  const int32_t* order;   // node slot b takes receiver order[b], or null
  int32_t x_dim, xoff, z_dim, zoff, c, cp;
  int32_t ls;
  int32_t accumulate;
  GeomParams g;
  CGTable cg;
};
hipError_t launch_fwd_uvu(const FwdUvuArgs& a, bool tangent, int li, int lo, int n_nodes, int ntiles, hipStream_t s);

// ---------------------------------------------------------------- backward, uvw
// One sender traversal for one path (Eq. 19-22 reassociated around the sender):
//   Q_e[w, m_in]  = sum_{m_out} cY_e[m_in, m_out] z_bar_i[w, m_out]
//   P_j[q, w, m_in] = sum_{e: j -> .} phi_q Q_e         (then x_bar = W^T P, W_bar = x^T P)
//   r_bar_e += d<z_bar, z>/dr_e using Xt_j = x_j W (radial and angular parts)
// With `tangent`: also dP_j = sum_e (dphi_q Q_e + phi_q dQ_e), dQ = cdY^T z_bar.
struct BwdUvwArgs {
  const int32_t* s_rowptr;
  const int32_t* s_col;
  const int32_t* s_slot;
  const float* pos;
  const float* pos_dot;   // tangent only
  const float* z_bar;
  const float* xt;        // [N*NI rows][ld_state]: Xt for this input block (needs_pos)
  float* P;               // [N*NI rows][ld_state] (needs_p)
  float* Pdot;            // tangent only
  float* rbar;            // [E][3] edge position adjoint, receiver-slot order (needs_pos)
  const int32_t* order;   // workgroup b takes sender order[b] (whole-graph launches), or null: send0 + b
  int32_t send0;          // first sender of this chunk (state rows are chunk-relative)
  int32_t z_dim, zoff, c_out, cp;
  int32_t ls;
  int64_t ld_state;       // floats per state row
  int32_t state_col0;     // column of (q = 0, w = 0) for this path
  int32_t rbar_accumulate;
  int32_t nparts;         // waves per channel tile that split a sender's edges (1..4)
  GeomParams g;
  CGTable cg;
};
// hess: position-Hessian pass of double backward (need_pos only): rbar receives the
// directional derivative of r_bar_e along r_dot_e = pos_dot_sender - pos_dot_receiver.
hipError_t launch_bwd_uvw(const BwdUvwArgs& a, bool need_p, bool need_pos, bool tangent, bool hess, int li, int lo,
                          int nsend, int ntiles, hipStream_t s);

// ---------------------------------------------------------------- backward, uvu
// Sender traversal for one uvu path: x_bar_j[u,m_in] (+)= sum_e w_e[u] Q_e[u,m_in];
// per-wave partial W_bar[q,u] = sum_e phi_q h_e[u], h = sum_m x_j Q; r_bar as above.
// With `tangent` (double backward along pos_dot): the same with w_e -> dw_e,
// Q -> dQ in the combinations of the VJP.
struct BwdUvuArgs {
  const int32_t* s_rowptr;
  const int32_t* s_col;
  const int32_t* s_slot;
  const float* pos;
  const float* pos_dot;
  const float* x;
  const float* w;         // path block [B][C]
  const float* z_bar;
  float* x_bar;           // [N][x_dim] or null
  float* wbar_part;       // [gridDim.x][B][C] per-block partial sums or null
  float* rbar;            // [E][3] or null
  int32_t n_nodes;
  int32_t x_dim, xoff, z_dim, zoff, c, cp;
  int32_t ls;
  int32_t xbar_accumulate, rbar_accumulate;
  GeomParams g;
  CGTable cg;
};
hipError_t launch_bwd_uvu(const BwdUvuArgs& a, bool tangent, bool hess, int li, int lo, int nblocks, int ntiles,
                          hipStream_t s);

// ---------------------------------------------------------------- dense fp32 GEMM on MFMA
// K slice of the 64 x 64 fp32 GEMM tiles (32 or 64; 64 measured 12-16% slower on the
// channel and node GEMMs: more LDS and registers per workgroup, fewer workgroups per
// CU); split-K ranges are multiples of it.
#ifndef ETPC_GEMM_BK
#define ETPC_GEMM_BK 32
#endif
constexpr int kGemmBK = ETPC_GEMM_BK;
// C(m, n) (+)= sum_k A(m, k) B(k, n)
//   a_mcontig = 0: A(m, k) = A[amap(m) + k];  1: A(m, k) = A[amap(k) + m]
//   B(k, n) = B[k * ldb + n];  C(m, n) = C[cmap(m) + n]
// Split-K: blockIdx.z handles K range [z*k_split, (z+1)*k_split) and writes its partial
// to C + z * c_split_stride (beta must then be 0).
struct GemmArgs {
  const float* A;
  RowMap amap;
  int32_t a_mcontig;
  const float* B;
  int64_t ldb;
  float* C;
  RowMap cmap;
  int32_t beta;
  int32_t M, N, K;
  int32_t k_split;
  int64_t c_split_stride;
  int32_t vec4;           // 1: every A row / B row start is 16-byte aligned (float4 loads allowed)
  int32_t lowp;           // operands rounded to 1: bf16, 2: fp16 (fp32 accumulation); 0: fp32
};
hipError_t launch_gemm(const GemmArgs& a, int splits, hipStream_t s);
// C(m, n) (+)= sum_{s < splits} part[s][m][n] (fixed order), C rows through cmap
hipError_t launch_splitk_reduce(const float* part, int splits, int M, int N, float* C, RowMap cmap, bool beta,
                                hipStream_t s);

// ---------------------------------------------------------------- small helpers
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s);
// W_bar scatter: out[path_off[t] + q*c_in*cout_t + u*cout_t + w] (+)= sum_{s < splits} part[s][u][col0_t + q*cout_t + w]
// (fixed summation order over the split-K partials; part rows have ncols columns).  While
// more than 64 copies remain, segments of 32 are summed in place, level by level, so part is
// clobbered.
hipError_t launch_reduce_wbar(float* part, int splits, int c_in, int n_paths, int nb, const int64_t* path_off,
                              const int32_t* col0, const int32_t* cout, int ncols, float* out, bool accumulate,
                              hipStream_t s);
// pos_bar[n] = sum_{sender slots of n} rbar[s_slot] - sum_{receiver slots of n} rbar[slot], where
// rbar[e] is the sum of `copies` arrays of n_edges x 3 floats (one per concurrent lane)
hipError_t launch_pos_bar(const int32_t* rowptr, const int32_t* s_rowptr, const int32_t* s_slot, const float* rbar,
                          int copies, int64_t n_edges, float* pos_bar, int n_nodes, hipStream_t s);
// Reorder W blocks of one input block into the layouts the node GEMMs read.
//   wcat[u][col0_t + q*cout_t + w]  = W_{pi_t}[q][u][w]   (t = position of the path within the input block)
//   wt[col0_t + q*cout_t + w][u]    = W_{pi_t}[q][u][w]
struct WPrepArgs {
  const float* w;
  float* wcat;
  float* wt;
  int64_t path_off[kMaxPaths];
  int32_t col0[kMaxPaths];
  int32_t cout[kMaxPaths];
  int32_t n_paths;
  int32_t nb, c_in, ncols;
};
hipError_t launch_wprep(const WPrepArgs& a, hipStream_t s);

}  // namespace etpc
