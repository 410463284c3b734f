// Forward receiver traversals (kernel templates; instantiated by fwd_*.hip).
//
// uvw: the receiver-factorized state of the Sobek paper (Sec. 4, Eq. 32-33).  One
// wavefront owns one receiver row of the receiver CSR.  Edge geometry is computed
// with one lane per incoming edge into LDS (radial basis phi_q and the contracted
// coupling cY[m_in][m_out] = sum_m_sh c[m_in][m_sh][m_out] Y[m_sh], which is
// channel independent); then each lane owns one input channel u, gathers the
// sender row x_j[u, :] (ir_mul: coalesced across lanes) and accumulates
//   S[q][m_out] += phi_q * sum_m_in x_j[u, m_in] cY[m_in][m_out]
// in registers.  Channel widths below 64 pack 64/cp edge slots into the wave;
// their partial states are summed with cross-lane shuffles at the end.
// S leaves the kernel as rows (i, m_out), columns (path, q, u): the A operand of
// the channel GEMM m = S W (Eq. 34-35).
//
// uvu: edge-local weight w_e[u] = sum_q phi_q W[q][u] (Eq. 17) applied in the same
// traversal; the output row is written directly (no channel GEMM for Eq. 7).
#pragma once
#include "cg_tables.inc"
#include "geom.hpp"
#include "kernels.hpp"
#include "triples.hpp"

namespace etpc {
namespace fwd_detail {

// sender-row gathers kept in flight per edge slot
#ifndef ETPC_FWD_PREFETCH
#define ETPC_FWD_PREFETCH 2
#endif
constexpr int kPrefetch = ETPC_FWD_PREFETCH;

// The state update S[q][m_out] += phi_q cm[m_out] on the matrix cores (1) or the VALU (0).
// As 4x4x1 blocks of four lanes: lane 4g + r supplies phi_{4qq+r}, every lane its own
// cm[m_out], so accumulator register r of a lane holds q = 4qq + r for its channel.
// Needs edge slots of at least four lanes (the host rounds the channel count up).
#ifndef ETPC_FWD_MFMA
#define ETPC_FWD_MFMA 1
#endif
constexpr bool kFwdMfma = ETPC_FWD_MFMA != 0;
// First-order uvu forward in the receiver-accumulated form (1) or the per-edge form (0).
// The accumulated form moves the per-edge coupling contraction to the matrix cores:
// channelwise workload, forward traversals 6.39 -> 5.46 ms per step.
#ifndef ETPC_FWD_UVU_ACC
#define ETPC_FWD_UVU_ACC 1
#endif
constexpr bool kFwdUvuAcc = ETPC_FWD_UVU_ACC != 0;
// Register budgets as resident waves per SIMD (0: the compiler's choice) of the
// accumulated uvu forward and of the uvw receiver traversal.  Both forwards measured
// slower with a budget (uvu at 3 waves: 5.38 -> 5.67 ms per step on the channelwise
// workload; uvw at 4 waves: 0.597 -> 0.614 ms on workload 2), unlike the uvu backward.
#ifndef ETPC_FWD_UVU_WAVES
#define ETPC_FWD_UVU_WAVES 0
#endif
#if ETPC_FWD_UVU_WAVES > 0
#define ETPC_FWD_UVU_ATTR __attribute__((amdgpu_waves_per_eu(ETPC_FWD_UVU_WAVES)))
#else
#define ETPC_FWD_UVU_ATTR
#endif
#ifndef ETPC_FWD_UVW_WAVES
#define ETPC_FWD_UVW_WAVES 0
#endif
#if ETPC_FWD_UVW_WAVES > 0
#define ETPC_FWD_UVW_ATTR __attribute__((amdgpu_waves_per_eu(ETPC_FWD_UVW_WAVES)))
#else
#define ETPC_FWD_UVW_ATTR
#endif
typedef float f4v __attribute__((ext_vector_type(4)));

// LDS per edge: phi[NB], (dphi[NB]), cY[NI*NO], (dcY[NI*NO]), padded by one float.
template <int NB, int CY, bool TANGENT>
struct EdgeLds {
  static constexpr int kPhi = 0;
  static constexpr int kPhiDot = NB;
  static constexpr int kCy = TANGENT ? 2 * NB : NB;
  static constexpr int kCyDot = kCy + CY;
  static constexpr int kStride = kCy + (TANGENT ? 2 * CY : CY) + 1;
};

// Fill one edge record (lane = edge).  j = sender, i = receiver.  cY (and its tangent)
// uses the compile-time sparse coupling table of (l_in, l_sh, l_out).
template <int LI, int LS, int LO, int NB, bool TANGENT>
__device__ inline void fill_edge(const GeomParams& g, const float* __restrict__ pos,
                                 const float* __restrict__ pos_dot, int j, int i, float* __restrict__ e) {
  constexpr int NI = 2 * LI + 1, NS = 2 * LS + 1, NO = 2 * LO + 1;
  using L = EdgeLds<NB, NI * NO, TANGENT>;
  using C = CgTab<LI, LS, LO>;
  float rx, ry, rz;
  edge_vector(g, pos, j, i, rx, ry, rz);
  const float r = sqrtf(rx * rx + ry * ry + rz * rz);
  const float ir = 1.f / r;
  const float ux = rx * ir, uy = ry * ir, uz = rz * ir;
  float phi[NB], dphi[NB];
  radial_eval<NB>(g, r, phi, TANGENT ? dphi : nullptr);
  float y[7];
  sh_eval(LS, ux, uy, uz, y);
#pragma unroll
  for (int q = 0; q < NB; ++q) e[L::kPhi + q] = phi[q];
  float ydot[7];
  if constexpr (TANGENT) {
    const float dx = pos_dot[3 * j + 0] - pos_dot[3 * i + 0];
    const float dy = pos_dot[3 * j + 1] - pos_dot[3 * i + 1];
    const float dz = pos_dot[3 * j + 2] - pos_dot[3 * i + 2];
    const float rdot = ux * dx + uy * dy + uz * dz;
#pragma unroll
    for (int q = 0; q < NB; ++q) e[L::kPhiDot + q] = dphi[q] * rdot;
    float gy[7][3];
    sh_grad_r(LS, ux, uy, uz, ir, y, gy);
#pragma unroll
    for (int m = 0; m < NS; ++m) ydot[m] = gy[m][0] * dx + gy[m][1] * dy + gy[m][2] * dz;
  }
#pragma unroll
  for (int a = 0; a < NI; ++a)
#pragma unroll
    for (int m = 0; m < NO; ++m) {
      float s = 0.f, sd = 0.f;
#pragma unroll
      for (int b = 0; b < NS; ++b) {
        if (C::v[a][b][m] != 0.f) {
          s += C::v[a][b][m] * y[b];
          if constexpr (TANGENT) sd += C::v[a][b][m] * ydot[b];
        }
      }
      e[L::kCy + a * NO + m] = s;
      if constexpr (TANGENT) e[L::kCyDot + a * NO + m] = sd;
    }
}

// SPLIT: a.nparts waves share the receiver's edges (small launches); without it the
// part count is the constant 1 and that code folds away.
template <int LI, int LS, int LO, int NBQ, bool TANGENT, bool SPLIT = false>
__global__ __launch_bounds__(SPLIT ? 256 : 64) ETPC_FWD_UVW_ATTR void fwd_uvw_kernel(const FwdUvwArgs a) {
  constexpr int NI = 2 * LI + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  using L = EdgeLds<NB, NI * NO, TANGENT>;
  __shared__ float s_edge[64 * L::kStride];
  __shared__ int s_j[64];
  extern __shared__ float s_part[];   // nparts > 1: accumulators handed to part 0
  const int lane = threadIdx.x & 63;
  const int part = SPLIT ? threadIdx.x >> 6 : 0;   // the wave's share of the receiver's edges
  const int nparts = SPLIT ? a.nparts : 1;
  // XCD-aware mapping of contiguous receiver ranges; with an order (heaviest first within
  // small aligned windows) each XCD still sweeps its own range, but every window ends on
  // short rows.  A receiver's S row does not depend on which workgroup takes it.
  const int nb = node_block(blockIdx.x, gridDim.x);
  const int bx = a.order ? a.order[nb] - a.recv0 : nb;
  const int i = a.recv0 + bx;
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  const int tslots = nslots * nparts;
  const int gslot = part * nslots + slot;
  const int u = blockIdx.y * cp + (lane - slot * cp);
  const bool uvalid = u < a.c_in;
  const int q4 = lane & 3;
  // acc[m_out][qq][r] = S[q = 4 qq + r][m_out] of the lane's channel
  f4v acc[NO][NBQ];
#pragma unroll
  for (int m = 0; m < NO; ++m)
#pragma unroll
    for (int qq = 0; qq < NBQ; ++qq) acc[m][qq] = f4v{0.f, 0.f, 0.f, 0.f};
  const int e0 = a.rowptr[i], e1 = a.rowptr[i + 1];
  for (int base = e0; base < e1; base += kWave) {
    const int ne = min(kWave, e1 - base);
    if (threadIdx.x < ne) {
      const int j = a.col[base + lane];
      fill_edge<LI, LS, LO, NB, TANGENT>(a.g, a.pos, a.pos_dot, j, i, s_edge + lane * L::kStride);
      s_j[lane] = j;
    }
    __syncthreads();
    const int trips = (ne + tslots - 1) / tslots;
    // sender rows of the next kPrefetch edges of this slot are in flight while one is used
    float xq[kPrefetch][NI];
    // Unconditional loads from a clamped in-bounds address (no branch per load); lanes
    // without an edge are zeroed when the row is consumed, not here, so nothing waits
    // on the load before its own trip.
    auto gather = [&](int t, float* dst) {
      const int j = s_j[t < ne ? t : 0];
      const float* xr = a.x + static_cast<int64_t>(t < ne ? j : 0) * a.x_dim + a.xoff + (uvalid ? u : 0);
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) dst[mi] = xr[mi * a.c_in];
    };
#pragma unroll
    for (int pf = 0; pf < kPrefetch; ++pf) {
      gather(pf * tslots + gslot, xq[pf]);
      // Pass the first rows through an arithmetic op: when every value entering the
      // loop-carried registers is a plain load, the optimizer merges them into one load
      // at the top of the loop, which undoes the prefetch.
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) xq[pf][mi] += 0.f;
    }
    for (int it0 = 0; it0 < trips; it0 += kPrefetch) {
#pragma unroll
      for (int pf = 0; pf < kPrefetch; ++pf) {
        // trips run in whole groups of kPrefetch (no exit inside the unrolled body, which
        // would make the compiler copy the loop-carried registers and wait on the loads);
        // a padding trip has t >= ne, gathers zeros and adds exact zeros
        const int it = it0 + pf;
        const int t = it * tslots + gslot;
        const float* e = s_edge + (t < ne ? t : 0) * L::kStride;
        const bool tv = t < ne && uvalid;
        float xv[NI];
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) xv[mi] = tv ? xq[pf][mi] : 0.f;
        float cm[NO], cmd[NO];
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) {
          float s = 0.f, sd = 0.f;
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) {
            s += xv[mi] * e[L::kCy + mi * NO + mo];
            if constexpr (TANGENT) sd += xv[mi] * e[L::kCyDot + mi * NO + mo];
          }
          cm[mo] = s;
          cmd[mo] = sd;
        }
        // the row is consumed: its registers take the gather kPrefetch trips ahead (no
        // register copy, so nothing waits for that load until its own trip); the
        // scheduling barrier keeps the loads here instead of sunk to the loop end
        gather(t + kPrefetch * tslots, xq[pf]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qq = 0; qq < NBQ; ++qq) {
          if constexpr (kFwdMfma) {
            const float ph = e[L::kPhi + 4 * qq + q4];
            const float phd = TANGENT ? e[L::kPhiDot + 4 * qq + q4] : 0.f;
#pragma unroll
            for (int mo = 0; mo < NO; ++mo) {
              if constexpr (TANGENT) {
                acc[mo][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(phd, cm[mo], acc[mo][qq], 0, 0, 0);
                acc[mo][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(ph, cmd[mo], acc[mo][qq], 0, 0, 0);
              } else {
                acc[mo][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(ph, cm[mo], acc[mo][qq], 0, 0, 0);
              }
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float ph = e[L::kPhi + 4 * qq + r];
              if constexpr (TANGENT) {
                const float phd = e[L::kPhiDot + 4 * qq + r];
#pragma unroll
                for (int mo = 0; mo < NO; ++mo) acc[mo][qq][r] += phd * cm[mo] + ph * cmd[mo];
              } else {
#pragma unroll
                for (int mo = 0; mo < NO; ++mo) acc[mo][qq][r] += ph * cm[mo];
              }
            }
          }
        }
      }
    }
    __syncthreads();
  }
  for (int off = cp; off < kWave; off <<= 1)
#pragma unroll
    for (int m = 0; m < NO; ++m)
#pragma unroll
      for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][qq][r] += __shfl_xor(acc[m][qq][r], off);
  for (int pp = 1; pp < nparts; ++pp) {
    // parts 1.. hand their sums to part 0 through LDS, one part at a time (fixed order)
    float* sx = s_part + lane * NB * NO;
    __syncthreads();
    if (part == pp && slot == 0)
#pragma unroll
      for (int m = 0; m < NO; ++m)
#pragma unroll
        for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
          for (int r = 0; r < 4; ++r) sx[(4 * qq + r) * NO + m] = acc[m][qq][r];
    __syncthreads();
    if (part == 0 && slot == 0)
#pragma unroll
      for (int m = 0; m < NO; ++m)
#pragma unroll
        for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[m][qq][r] += sx[(4 * qq + r) * NO + m];
  }
  if (part == 0 && slot == 0 && uvalid) {
    float* srow = a.S + static_cast<int64_t>(bx) * NO * a.s_row_stride + a.s_col0 + u;
#pragma unroll
    for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * qq + r < a.g.nb)
#pragma unroll
          for (int mo = 0; mo < NO; ++mo) srow[mo * a.s_row_stride + (4 * qq + r) * a.c_in] = acc[mo][qq][r];
  }
}

template <int LI, int LS, int LO, int NBQ, bool TANGENT>
__global__ __launch_bounds__(64) void fwd_uvu_kernel(const FwdUvuArgs a) {
  constexpr int NI = 2 * LI + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  using L = EdgeLds<NB, NI * NO, TANGENT>;
  __shared__ float s_edge[64 * L::kStride];
  __shared__ int s_j[64];
  const int lane = threadIdx.x;
  // XCD-aware slots, then the receiver order within small windows (as in the uvw traversal)
  const int nb = node_block(blockIdx.x, gridDim.x);
  const int i = a.order ? a.order[nb] : nb;
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  const int u = blockIdx.y * cp + (lane - slot * cp);
  const bool uvalid = u < a.c;
  float wv[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) wv[q] = (uvalid && q < a.g.nb) ? a.w[q * a.c + u] : 0.f;
  float acc[NO];
#pragma unroll
  for (int m = 0; m < NO; ++m) acc[m] = 0.f;
  const int e0 = a.rowptr[i], e1 = a.rowptr[i + 1];
  for (int base = e0; base < e1; base += kWave) {
    const int ne = min(kWave, e1 - base);
    if (lane < ne) {
      const int j = a.col[base + lane];
      fill_edge<LI, LS, LO, NB, TANGENT>(a.g, a.pos, a.pos_dot, j, i, s_edge + lane * L::kStride);
      s_j[lane] = j;
    }
    __syncthreads();
    const int trips = (ne + nslots - 1) / nslots;
    float xq[kPrefetch][NI];
    // same software pipeline as the uvw traversal: clamped unconditional loads, rows
    // zeroed when consumed, whole groups of kPrefetch trips
    auto gather = [&](int t, float* dst) {
      const int j = s_j[t < ne ? t : 0];
      const float* xr = a.x + static_cast<int64_t>(t < ne ? j : 0) * a.x_dim + a.xoff + (uvalid ? u : 0);
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) dst[mi] = xr[mi * a.c];
    };
#pragma unroll
    for (int pf = 0; pf < kPrefetch; ++pf) {
      gather(pf * nslots + slot, xq[pf]);
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) xq[pf][mi] += 0.f;   // not a plain load (see above)
    }
    for (int it0 = 0; it0 < trips; it0 += kPrefetch) {
#pragma unroll
      for (int pf = 0; pf < kPrefetch; ++pf) {
        const int t = (it0 + pf) * nslots + slot;
        const bool tv = t < ne && uvalid;
        const float* e = s_edge + (t < ne ? t : 0) * L::kStride;
        float xv[NI];
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) xv[mi] = tv ? xq[pf][mi] : 0.f;
        gather(t + kPrefetch * nslots, xq[pf]);
        __builtin_amdgcn_sched_barrier(0);
        float we = 0.f, wed = 0.f;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          we += e[L::kPhi + q] * wv[q];
          if constexpr (TANGENT) wed += e[L::kPhiDot + q] * wv[q];
        }
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) {
          float s = 0.f, sd = 0.f;
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) {
            s += xv[mi] * e[L::kCy + mi * NO + mo];
            if constexpr (TANGENT) sd += xv[mi] * e[L::kCyDot + mi * NO + mo];
          }
          if constexpr (TANGENT)
            acc[mo] += wed * s + we * sd;
          else
            acc[mo] += we * s;
        }
      }
    }
    __syncthreads();
  }
  for (int off = cp; off < kWave; off <<= 1)
#pragma unroll
    for (int m = 0; m < NO; ++m) acc[m] += __shfl_xor(acc[m], off);
  if (slot == 0 && uvalid) {
    float* zr = a.z + static_cast<int64_t>(i) * a.z_dim + a.zoff + u;
#pragma unroll
    for (int mo = 0; mo < NO; ++mo) {
      if (a.accumulate)
        zr[mo * a.c] += acc[mo];
      else
        zr[mo * a.c] = acc[mo];
    }
  }
}

// uvu forward with the edge sum regrouped around the receiver (first order).  With c the
// path's coupling tensor, for lane channel u of receiver i:
//   z_i[m] = sum_e w_e sum_{a,b} c[a][b][m] x_j[a] Y_e[b] = sum_{a,b} c[a][b][m] A_i[b][a],
//   A_i[b][a] = sum_e Y_e[b] (w_e x_j[a])
// (Eq. 7 with the edge-local weight of Eq. 17, reassociated; exact in exact arithmetic).
// A_i accumulates on the matrix cores as 4x4x1 blocks of four lanes: lane 4g + r supplies
// Y[4k + r] of the edge, every lane its own w_e x_j[a], so register r of Ac[k][a] holds
// b = 4k + r.  The radial weights w_e = sum_q phi_q W[q][u] of four trips come from the
// same blocks (row r takes phi of trip it0 + r, each lane's column its W[q][u]).  The
// edge record shrinks to phi and the zero-padded harmonics; the coupling is applied once
// per receiver.
template <int NB, int NSQ>
struct EdgeLdsY {
  static constexpr int kPhi = 0;
  static constexpr int kY = NB;
  static constexpr int kStride = NB + 4 * NSQ + 1;   // odd: the four records a block reads sit in four banks
};

template <int LS, int NB, int NSQ>
__device__ inline void fill_edge_y(const GeomParams& g, const float* __restrict__ pos, int j, int i,
                                   float* __restrict__ e) {
  using L = EdgeLdsY<NB, NSQ>;
  float rx, ry, rz;
  edge_vector(g, pos, j, i, rx, ry, rz);
  const float r = sqrtf(rx * rx + ry * ry + rz * rz);
  const float ir = 1.f / r;
  float phi[NB];
  radial_eval<NB>(g, r, phi, nullptr);
  float y[7];
  sh_eval(LS, rx * ir, ry * ir, rz * ir, y);
#pragma unroll
  for (int q = 0; q < NB; ++q) e[L::kPhi + q] = phi[q];
#pragma unroll
  for (int b = 0; b < 4 * NSQ; ++b) e[L::kY + b] = b < 2 * LS + 1 ? y[b] : 0.f;
}

template <int LI, int LS, int LO, int NBQ>
__global__ __launch_bounds__(64) ETPC_FWD_UVU_ATTR void fwd_uvu_acc_kernel(const FwdUvuArgs a) {
  constexpr int NI = 2 * LI + 1, NS = 2 * LS + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  constexpr int NSQ = (NS + 3) / 4;
  constexpr int kGroup = 4;   // trips per radial-weight group; also the gather distance
  using L = EdgeLdsY<NB, NSQ>;
  using C = CgTab<LI, LS, LO>;
  __shared__ float s_edge[64 * L::kStride];
  __shared__ int s_j[64];
  const int lane = threadIdx.x;
  const int nb = node_block(blockIdx.x, gridDim.x);
  const int i = a.order ? a.order[nb] : nb;
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  const int u = blockIdx.y * cp + (lane - slot * cp);
  const bool uvalid = u < a.c;
  const int q4 = lane & 3;
  float wv[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) wv[q] = (uvalid && q < a.g.nb) ? a.w[q * a.c + u] : 0.f;
  f4v Ac[NSQ][NI];
#pragma unroll
  for (int k = 0; k < NSQ; ++k)
#pragma unroll
    for (int mi = 0; mi < NI; ++mi) Ac[k][mi] = f4v{0.f, 0.f, 0.f, 0.f};
  const int e0 = a.rowptr[i], e1 = a.rowptr[i + 1];
  for (int base = e0; base < e1; base += kWave) {
    const int ne = min(kWave, e1 - base);
    if (lane < ne) {
      const int j = a.col[base + lane];
      fill_edge_y<LS, NB, NSQ>(a.g, a.pos, j, i, s_edge + lane * L::kStride);
      s_j[lane] = j;
    }
    __syncthreads();
    const int trips = (ne + nslots - 1) / nslots;
    float xq[kGroup][NI];
    // clamped unconditional loads (lanes past c read channel 0 and are weighted by W = 0)
    auto gather = [&](int t, float* dst) {
      const int j = s_j[t < ne ? t : 0];
      const float* xr = a.x + static_cast<int64_t>(t < ne ? j : 0) * a.x_dim + a.xoff + (uvalid ? u : 0);
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) dst[mi] = xr[mi * a.c];
    };
#pragma unroll
    for (int pf = 0; pf < kGroup; ++pf) {
      gather(pf * nslots + slot, xq[pf]);
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) xq[pf][mi] += 0.f;   // not a plain load (see the uvw traversal)
    }
    for (int it0 = 0; it0 < trips; it0 += kGroup) {
      // w_e of trips it0 .. it0 + 3 for the lane's channel (register r: trip it0 + r)
      const int tt = (it0 + q4) * nslots + slot;
      const float* er = s_edge + (tt < ne ? tt : 0) * L::kStride + L::kPhi;
      f4v WE = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < NB; ++q) WE = __builtin_amdgcn_mfma_f32_4x4x1f32(er[q], wv[q], WE, 0, 0, 0);
#pragma unroll
      for (int pf = 0; pf < kGroup; ++pf) {
        const int t = (it0 + pf) * nslots + slot;
        const bool tv = t < ne;
        // a padding trip (t >= ne) reads edge 0's record and a clamped row with weight 0
        const float we = tv ? WE[pf] : 0.f;
        float tx[NI];
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) tx[mi] = we * xq[pf][mi];
        gather(t + kGroup * nslots, xq[pf]);
        __builtin_amdgcn_sched_barrier(0);
        const float* e = s_edge + (tv ? t : 0) * L::kStride + L::kY;
#pragma unroll
        for (int k = 0; k < NSQ; ++k) {
          const float yv = e[4 * k + q4];
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) Ac[k][mi] = __builtin_amdgcn_mfma_f32_4x4x1f32(yv, tx[mi], Ac[k][mi], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  float acc[NO];
#pragma unroll
  for (int mo = 0; mo < NO; ++mo) {
    float s = 0.f;
#pragma unroll
    for (int mi = 0; mi < NI; ++mi)
#pragma unroll
      for (int b = 0; b < NS; ++b)
        if (C::v[mi][b][mo] != 0.f) s += C::v[mi][b][mo] * Ac[b / 4][mi][b % 4];
    acc[mo] = s;
  }
  for (int off = cp; off < kWave; off <<= 1)
#pragma unroll
    for (int m = 0; m < NO; ++m) acc[m] += __shfl_xor(acc[m], off);
  if (slot == 0 && uvalid) {
    float* zr = a.z + static_cast<int64_t>(i) * a.z_dim + a.zoff + u;
#pragma unroll
    for (int mo = 0; mo < NO; ++mo) {
      if (a.accumulate)
        zr[mo * a.c] += acc[mo];
      else
        zr[mo * a.c] = acc[mo];
    }
  }
}

template <int LI, int LS, int LO, bool T>
hipError_t fwd_uvw_nb(const FwdUvwArgs& a, int nrecv, int ntiles, hipStream_t s) {
  dim3 grid(nrecv, ntiles), block(64 * a.nparts);
  const size_t dyn = a.nparts > 1 ? sizeof(float) * 64 * (2 * LO + 1) * (a.g.nb <= 8 ? 8 : 16) : 0;
  const bool split = a.nparts > 1;
  if (a.g.nb <= 8) {
    if (split)
      hipLaunchKernelGGL((fwd_uvw_kernel<LI, LS, LO, 2, T, true>), grid, block, dyn, s, a);
    else
      hipLaunchKernelGGL((fwd_uvw_kernel<LI, LS, LO, 2, T, false>), grid, block, dyn, s, a);
  } else {
    if (split)
      hipLaunchKernelGGL((fwd_uvw_kernel<LI, LS, LO, 4, T, true>), grid, block, dyn, s, a);
    else
      hipLaunchKernelGGL((fwd_uvw_kernel<LI, LS, LO, 4, T, false>), grid, block, dyn, s, a);
  }
  return hipGetLastError();
}

template <int LI, int LS, int LO, bool T>
hipError_t fwd_uvu_nb(const FwdUvuArgs& a, int n, int ntiles, hipStream_t s) {
  dim3 grid(n, ntiles), block(64);
  if constexpr (!T && kFwdUvuAcc) {
    if (a.g.nb <= 8)
      hipLaunchKernelGGL((fwd_uvu_acc_kernel<LI, LS, LO, 2>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_uvu_acc_kernel<LI, LS, LO, 4>), grid, block, 0, s, a);
  } else {
    if (a.g.nb <= 8)
      hipLaunchKernelGGL((fwd_uvu_kernel<LI, LS, LO, 2, T>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_uvu_kernel<LI, LS, LO, 4, T>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <bool T>
hipError_t launch_fwd_uvw_t(const FwdUvwArgs& a, int li, int lo, int nrecv, int ntiles, hipStream_t s) {
#define ETPC_CALL(LI, LS, LO) fwd_uvw_nb<LI, LS, LO, T>(a, nrecv, ntiles, s)
  ETPC_TRIPLE_DISPATCH(li, a.ls, lo, ETPC_CALL)
#undef ETPC_CALL
}

template <bool T>
hipError_t launch_fwd_uvu_t(const FwdUvuArgs& a, int li, int lo, int n, int ntiles, hipStream_t s) {
#define ETPC_CALL(LI, LS, LO) fwd_uvu_nb<LI, LS, LO, T>(a, n, ntiles, s)
  ETPC_TRIPLE_DISPATCH(li, a.ls, lo, ETPC_CALL)
#undef ETPC_CALL
}

}  // namespace fwd_detail
}  // namespace etpc
