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
#include "geom.hpp"
#include "kernels.hpp"

namespace etpc {
namespace fwd_detail {

// LDS per edge: phi[NB], (dphi[NB]), cY[NI*NO], (dcY[NI*NO]), padded by one float.
template <int NB, int CY, bool TANGENT>
struct EdgeLds {
  static constexpr int kPhi = 0;
  static constexpr int kPhiDot = NB;
  static constexpr int kCy = TANGENT ? 2 * NB : NB;
  static constexpr int kCyDot = kCy + CY;
  static constexpr int kStride = kCy + (TANGENT ? 2 * CY : CY) + 1;
};

// Fill one edge record (lane = edge).  j = sender, i = receiver.
template <int NI, int NO, int NB, bool TANGENT>
__device__ inline void fill_edge(const GeomParams& g, const CGTable& cg, int ls, const float* __restrict__ pos,
                                 const float* __restrict__ pos_dot, int j, int i, float* __restrict__ e) {
  using L = EdgeLds<NB, NI * NO, TANGENT>;
  float rx, ry, rz;
  edge_vector(g, pos, j, i, rx, ry, rz);
  const float r = sqrtf(rx * rx + ry * ry + rz * rz);
  const float ir = 1.f / r;
  const float ux = rx * ir, uy = ry * ir, uz = rz * ir;
  float phi[NB], dphi[NB];
  radial_eval<NB>(g, r, phi, TANGENT ? dphi : nullptr);
  float y[7];
  sh_eval(ls, ux, uy, uz, y);
  const int nsh = 2 * ls + 1;
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
    sh_grad_r(ls, ux, uy, uz, ir, y, gy);
    for (int m = 0; m < nsh; ++m) ydot[m] = gy[m][0] * dx + gy[m][1] * dy + gy[m][2] * dz;
  }
#pragma unroll
  for (int a = 0; a < NI; ++a)
#pragma unroll
    for (int m = 0; m < NO; ++m) {
      float s = 0.f, sd = 0.f;
      for (int b = 0; b < nsh; ++b) {
        const float c = cg.c[(a * 7 + b) * NO + m];
        s += c * y[b];
        if constexpr (TANGENT) sd += c * ydot[b];
      }
      e[L::kCy + a * NO + m] = s;
      if constexpr (TANGENT) e[L::kCyDot + a * NO + m] = sd;
    }
}

typedef float f4v __attribute__((ext_vector_type(4)));

// The radial outer product S[q][m_out] += phi_q C[m_out] runs on the matrix cores:
// v_mfma_f32_4x4x1f32 with A = phi[4 qq + (lane & 3)] (per-lane LDS read) and
// B = C[m_out] of the lane's channel gives, in lane l and register r, phi[4 qq + r] C_l[m_out],
// i.e. each lane accumulates its own channel's S[4 qq .. 4 qq + 3][m_out].
template <int LI, int LO, int NBQ, bool TANGENT>
__global__ __launch_bounds__(64, 3) void fwd_uvw_kernel(const FwdUvwArgs a) {
  constexpr int NI = 2 * LI + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  using L = EdgeLds<NB, NI * NO, TANGENT>;
  __shared__ float s_edge[64 * L::kStride];
  __shared__ int s_j[64];
  const int lane = threadIdx.x;
  const int i = a.recv0 + blockIdx.x;
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  const int u = blockIdx.y * cp + (lane - slot * cp);
  const bool uvalid = u < a.c_in;
  const int q4 = lane & 3;
  f4v acc[NO][NBQ];
#pragma unroll
  for (int m = 0; m < NO; ++m)
#pragma unroll
    for (int qq = 0; qq < NBQ; ++qq) acc[m][qq] = f4v{0.f, 0.f, 0.f, 0.f};
  const int e0 = a.rowptr[i], e1 = a.rowptr[i + 1];
  for (int base = e0; base < e1; base += kWave) {
    const int ne = min(kWave, e1 - base);
    if (lane < ne) {
      const int j = a.col[base + lane];
      fill_edge<NI, NO, NB, TANGENT>(a.g, a.cg, a.ls, a.pos, a.pos_dot, j, i, s_edge + lane * L::kStride);
      s_j[lane] = j;
    }
    __syncthreads();
    const int trips = (ne + nslots - 1) / nslots;
    // gathered sender rows, one edge ahead (zero for lanes without a channel or an edge)
    float xn[NI];
    {
      const bool v = uvalid && slot < ne;
      const float* xr = a.x + static_cast<int64_t>(v ? s_j[slot] : 0) * a.x_dim + a.xoff + u;
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) xn[mi] = v ? xr[mi * a.c_in] : 0.f;
    }
    for (int it = 0; it < trips; ++it) {
      const int t = it * nslots + slot;
      const bool tvalid = t < ne;
      const float* e = s_edge + (tvalid ? t : 0) * L::kStride;
      float xv[NI];
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) xv[mi] = xn[mi];
      {
        const int tn = t + nslots;
        const bool v = uvalid && tn < ne;
        const float* xr = a.x + static_cast<int64_t>(v ? s_j[tn] : 0) * a.x_dim + a.xoff + u;
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) xn[mi] = v ? xr[mi * a.c_in] : 0.f;
      }
      float cm[NO], cmd[NO];
#pragma unroll
      for (int mo = 0; mo < NO; ++mo) {
        float s = 0.f, sd = 0.f;
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) {
          s += xv[mi] * e[L::kCy + mi * NO + mo];
          if constexpr (TANGENT) sd += xv[mi] * e[L::kCyDot + mi * NO + mo];
        }
        cm[mo] = tvalid ? s : 0.f;
        cmd[mo] = tvalid ? sd : 0.f;
      }
#pragma unroll
      for (int qq = 0; qq < NBQ; ++qq) {
        const float ph = e[L::kPhi + 4 * qq + q4];
        if constexpr (TANGENT) {
          const float phd = e[L::kPhiDot + 4 * qq + q4];
#pragma unroll
          for (int mo = 0; mo < NO; ++mo) {
            acc[mo][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(phd, cm[mo], acc[mo][qq], 0, 0, 0);
            acc[mo][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(ph, cmd[mo], acc[mo][qq], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int mo = 0; mo < NO; ++mo)
            acc[mo][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(ph, cm[mo], acc[mo][qq], 0, 0, 0);
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
  if (slot == 0 && uvalid) {
    float* srow = a.S + static_cast<int64_t>(blockIdx.x) * NO * a.s_row_stride + a.s_col0 + u;
#pragma unroll
    for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * qq + r < a.g.nb)
#pragma unroll
          for (int mo = 0; mo < NO; ++mo) srow[mo * a.s_row_stride + (4 * qq + r) * a.c_in] = acc[mo][qq][r];
  }
}

template <int LI, int LO, int NBQ, bool TANGENT>
__global__ __launch_bounds__(64) void fwd_uvu_kernel(const FwdUvuArgs a) {
  constexpr int NI = 2 * LI + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  using L = EdgeLds<NB, NI * NO, TANGENT>;
  __shared__ float s_edge[64 * L::kStride];
  __shared__ int s_j[64];
  const int lane = threadIdx.x;
  const int i = blockIdx.x;
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
      fill_edge<NI, NO, NB, TANGENT>(a.g, a.cg, a.ls, a.pos, a.pos_dot, j, i, s_edge + lane * L::kStride);
      s_j[lane] = j;
    }
    __syncthreads();
    if (uvalid && slot < ne) {
      float xn[NI];
      {
        const float* xr = a.x + static_cast<int64_t>(s_j[slot]) * a.x_dim + a.xoff + u;
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) xn[mi] = xr[mi * a.c];
      }
      for (int t = slot; t < ne; t += nslots) {
        const float* e = s_edge + t * L::kStride;
        float xv[NI];
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) xv[mi] = xn[mi];
        if (t + nslots < ne) {
          const float* xr = a.x + static_cast<int64_t>(s_j[t + nslots]) * a.x_dim + a.xoff + u;
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) xn[mi] = xr[mi * a.c];
        }
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

template <int LI, int LO, bool T>
hipError_t fwd_uvw_nb(const FwdUvwArgs& a, int nrecv, int ntiles, hipStream_t s) {
  dim3 grid(nrecv, ntiles), block(64);
  switch ((a.g.nb + 3) / 4) {
    case 1: hipLaunchKernelGGL((fwd_uvw_kernel<LI, LO, 1, T>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((fwd_uvw_kernel<LI, LO, 2, T>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((fwd_uvw_kernel<LI, LO, 3, T>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((fwd_uvw_kernel<LI, LO, 4, T>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int LI, int LO, bool T>
hipError_t fwd_uvu_nb(const FwdUvuArgs& a, int n, int ntiles, hipStream_t s) {
  dim3 grid(n, ntiles), block(64);
  switch ((a.g.nb + 3) / 4) {
    case 1: hipLaunchKernelGGL((fwd_uvu_kernel<LI, LO, 1, T>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((fwd_uvu_kernel<LI, LO, 2, T>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((fwd_uvu_kernel<LI, LO, 3, T>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((fwd_uvu_kernel<LI, LO, 4, T>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

#define ETPC_LL_SWITCH(FN, T, ...)                 \
  switch (li * 4 + lo) {                           \
    case 0: return FN<0, 0, T>(__VA_ARGS__);       \
    case 1: return FN<0, 1, T>(__VA_ARGS__);       \
    case 2: return FN<0, 2, T>(__VA_ARGS__);       \
    case 3: return FN<0, 3, T>(__VA_ARGS__);       \
    case 4: return FN<1, 0, T>(__VA_ARGS__);       \
    case 5: return FN<1, 1, T>(__VA_ARGS__);       \
    case 6: return FN<1, 2, T>(__VA_ARGS__);       \
    case 7: return FN<1, 3, T>(__VA_ARGS__);       \
    case 8: return FN<2, 0, T>(__VA_ARGS__);       \
    case 9: return FN<2, 1, T>(__VA_ARGS__);       \
    case 10: return FN<2, 2, T>(__VA_ARGS__);      \
    case 11: return FN<2, 3, T>(__VA_ARGS__);      \
    case 12: return FN<3, 0, T>(__VA_ARGS__);      \
    case 13: return FN<3, 1, T>(__VA_ARGS__);      \
    case 14: return FN<3, 2, T>(__VA_ARGS__);      \
    default: return FN<3, 3, T>(__VA_ARGS__);      \
  }

template <bool T>
hipError_t launch_fwd_uvw_t(const FwdUvwArgs& a, int li, int lo, int nrecv, int ntiles, hipStream_t s) {
  ETPC_LL_SWITCH(fwd_uvw_nb, T, a, nrecv, ntiles, s)
}

template <bool T>
hipError_t launch_fwd_uvu_t(const FwdUvuArgs& a, int li, int lo, int n, int ntiles, hipStream_t s) {
  ETPC_LL_SWITCH(fwd_uvu_nb, T, a, n, ntiles, s)
}

}  // namespace fwd_detail
}  // namespace etpc
