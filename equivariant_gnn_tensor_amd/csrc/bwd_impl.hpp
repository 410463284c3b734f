// Backward sender traversals (kernel templates; instantiated by bwd_*.hip).
//
// The Sobek paper's first-order adjoints (Sec. 3, Eq. 18-22) are all edge local.
// Its execution architecture (Sec. 4) owns x_bar by a source-contiguous CSR
// traversal with one fixed reduction order.  Here the whole backward of a path is
// one such sender traversal: for sender j and each outgoing edge e = (j -> i),
//   Q_e[w, m_in]  = sum_m_out cY_e[m_in, m_out] z_bar_i[w, m_out]         (gathered z_bar row)
//   P_j[q, w, m_in] += phi_q(r_e) Q_e[w, m_in]                             (sender state, no u axis)
//   phi_bar_e[q]  = sum_{w, m_in} Xt_j[q, w, m_in] Q_e[w, m_in]            (Eq. 20, Xt = x W)
//   Y_bar_e       = sum c (sum_q phi_q Xt_j[q]) (x) z_bar_i                 (Eq. 22)
// and the two edge adjoints are folded at once into the edge-vector adjoint
//   r_bar_e = u sum_q phi'_q phi_bar_q + sum_m dY_m/dr_e Y_bar_m          (chain rule through Eq. 8)
// which is the only per-edge value that leaves the kernel (3 floats, receiver-slot
// order).  x_bar = W^T P and W_bar = x^T P (Eq. 19, 21) then run on the matrix
// cores.  The double-backward tangent along pos_dot adds
//   dP_j = sum_e (dphi_q Q_e + phi_q dQ_e),  dQ = cdY^T z_bar,
// the differentiated receiver program of Eq. 37-39 seen from the sender side.
//
// uvu (Eq. 7): per lane channel u, w_e[u] = sum_q phi_q W[q, u] (Eq. 17),
//   x_bar_j[u] += w_e Q_e,  h_e[u] = <x_j[u], Q_e[u]>,  W_bar[q, u] += phi_q h_e,
// W_bar kept as per-workgroup partials (fixed sender ranges, fixed-order reduction).
#pragma once
#include "geom.hpp"
#include "kernels.hpp"

namespace etpc {
namespace bwd_detail {

constexpr int kMaxTiles = 4;

// LDS edge record offsets
template <int NB, int NI, int NO, bool POS, bool TAN>
struct BwdLds {
  static constexpr int CY = NI * NO;
  static constexpr int kPhi = 0;
  static constexpr int kDphi = NB;                       // radial derivative (POS)
  static constexpr int kPhiDot = 2 * NB;                 // tangent
  static constexpr int kCy = 3 * NB;
  static constexpr int kCdy = kCy + CY;                  // 3 x CY (POS)
  static constexpr int kCyDot = kCdy + 3 * CY;           // tangent
  static constexpr int kU = kCyDot + CY;                 // unit vector (POS)
  static constexpr int kStride = kU + 3 + 1;
};

template <int NB, int NI, int NO, bool POS, bool TAN>
__device__ inline void bwd_fill_edge(const GeomParams& g, const CGTable& cg, int ls, const float* __restrict__ pos,
                                     const float* __restrict__ pos_dot, int j, int i, float* __restrict__ e) {
  using L = BwdLds<NB, NI, NO, POS, TAN>;
  float rx, ry, rz;
  edge_vector(g, pos, j, i, rx, ry, rz);
  const float r = sqrtf(rx * rx + ry * ry + rz * rz);
  const float ir = 1.f / r;
  const float ux = rx * ir, uy = ry * ir, uz = rz * ir;
  constexpr bool NEED_D = POS || TAN;
  float phi[NB], dphi[NB];
  radial_eval<NB>(g, r, phi, NEED_D ? dphi : nullptr);
  float y[7];
  sh_eval(ls, ux, uy, uz, y);
  const int nsh = 2 * ls + 1;
  float gy[7][3];
  if constexpr (NEED_D) sh_grad_r(ls, ux, uy, uz, ir, y, gy);
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    e[L::kPhi + q] = phi[q];
    if constexpr (POS) e[L::kDphi + q] = dphi[q];
  }
  float ydot[7];
  if constexpr (TAN) {
    const float dx = pos_dot[3 * j + 0] - pos_dot[3 * i + 0];
    const float dy = pos_dot[3 * j + 1] - pos_dot[3 * i + 1];
    const float dz = pos_dot[3 * j + 2] - pos_dot[3 * i + 2];
    const float rdot = ux * dx + uy * dy + uz * dz;
#pragma unroll
    for (int q = 0; q < NB; ++q) e[L::kPhiDot + q] = dphi[q] * rdot;
    for (int m = 0; m < nsh; ++m) ydot[m] = gy[m][0] * dx + gy[m][1] * dy + gy[m][2] * dz;
  }
  if constexpr (POS) {
    e[L::kU + 0] = ux;
    e[L::kU + 1] = uy;
    e[L::kU + 2] = uz;
  }
#pragma unroll
  for (int a = 0; a < NI; ++a)
#pragma unroll
    for (int m = 0; m < NO; ++m) {
      float s = 0.f, s0 = 0.f, s1 = 0.f, s2 = 0.f, sd = 0.f;
      for (int b = 0; b < nsh; ++b) {
        const float c = cg.c[(a * 7 + b) * NO + m];
        s += c * y[b];
        if constexpr (POS) {
          s0 += c * gy[b][0];
          s1 += c * gy[b][1];
          s2 += c * gy[b][2];
        }
        if constexpr (TAN) sd += c * ydot[b];
      }
      e[L::kCy + a * NO + m] = s;
      if constexpr (POS) {
        e[L::kCdy + a * NO + m] = s0;
        e[L::kCdy + L::CY + a * NO + m] = s1;
        e[L::kCdy + 2 * L::CY + a * NO + m] = s2;
      }
      if constexpr (TAN) e[L::kCyDot + a * NO + m] = sd;
    }
}

// sum over the cp lanes of one slot (cp a power of two); every lane of the slot gets the sum
__device__ inline float slot_sum(float v, int cp) {
  for (int off = 1; off < cp; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

template <int LI, int LO, int NBQ, bool NEED_P, bool POS, bool TAN>
__global__ __launch_bounds__(256) void bwd_uvw_kernel(const BwdUvwArgs a) {
  constexpr int NI = 2 * LI + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  using L = BwdLds<NB, NI, NO, POS, TAN>;
  __shared__ float s_edge[64 * L::kStride];
  __shared__ int s_i[64];
  __shared__ int s_sl[64];
  __shared__ float s_rb[kMaxTiles][64][3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int j = a.send0 + blockIdx.x;
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  const int w = wave * cp + (lane - slot * cp);
  const bool wvalid = w < a.c_out;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * NI;
  float xt[NB][NI];
  if constexpr (POS) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int mi = 0; mi < NI; ++mi)
        xt[q][mi] = (wvalid && q < a.g.nb)
                        ? a.xt[(row0 + mi) * a.ld_state + a.state_col0 + static_cast<int64_t>(q) * a.c_out + w]
                        : 0.f;
  }
  float P[NB][NI], Pd[NB][NI];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int mi = 0; mi < NI; ++mi) {
      P[q][mi] = 0.f;
      Pd[q][mi] = 0.f;
    }
  const int k0 = a.s_rowptr[j], k1 = a.s_rowptr[j + 1];
  for (int base = k0; base < k1; base += kWave) {
    const int ne = min(kWave, k1 - base);
    if (tid < ne) {
      const int i = a.s_col[base + tid];
      bwd_fill_edge<NB, NI, NO, POS, TAN>(a.g, a.cg, a.ls, a.pos, a.pos_dot, j, i, s_edge + tid * L::kStride);
      s_i[tid] = i;
      s_sl[tid] = a.s_slot[base + tid];
    }
    __syncthreads();
    const int trips = (ne + nslots - 1) / nslots;
    for (int it = 0; it < trips; ++it) {
      const int t = it * nslots + slot;
      const bool tvalid = t < ne;
      const float* e = s_edge + (tvalid ? t : 0) * L::kStride;
      float zb[NO];
      const float* zr = a.z_bar + static_cast<int64_t>(tvalid ? s_i[t] : 0) * a.z_dim + a.zoff + w;
#pragma unroll
      for (int mo = 0; mo < NO; ++mo) zb[mo] = (tvalid && wvalid) ? zr[mo * a.c_out] : 0.f;
      float Q[NI], Qd[NI];
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) {
        float s = 0.f, sd = 0.f;
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) {
          s += e[L::kCy + mi * NO + mo] * zb[mo];
          if constexpr (TAN) sd += e[L::kCyDot + mi * NO + mo] * zb[mo];
        }
        Q[mi] = s;
        Qd[mi] = sd;
      }
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const float ph = e[L::kPhi + q];
        if constexpr (NEED_P) {
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) P[q][mi] += ph * Q[mi];
        }
        if constexpr (TAN) {
          const float phd = e[L::kPhiDot + q];
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) Pd[q][mi] += phd * Q[mi] + ph * Qd[mi];
        }
      }
      if constexpr (POS) {
        float srad = 0.f;
        float T[NI];
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) {
          float gq = 0.f, tq = 0.f;
#pragma unroll
          for (int q = 0; q < NB; ++q) {
            gq += e[L::kDphi + q] * xt[q][mi];
            tq += e[L::kPhi + q] * xt[q][mi];
          }
          srad += gq * Q[mi];
          T[mi] = tq;
        }
        float rb[3];
#pragma unroll
        for (int d = 0; d < 3; ++d) {
          float s = 0.f;
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) {
            float zc = 0.f;
#pragma unroll
            for (int mo = 0; mo < NO; ++mo) zc += e[L::kCdy + d * L::CY + mi * NO + mo] * zb[mo];
            s += T[mi] * zc;
          }
          rb[d] = slot_sum(srad * e[L::kU + d] + s, cp);
        }
        if (tvalid && lane == slot * cp) {
          s_rb[wave][t][0] = rb[0];
          s_rb[wave][t][1] = rb[1];
          s_rb[wave][t][2] = rb[2];
        }
      }
    }
    __syncthreads();
    if constexpr (POS) {
      if (tid < ne) {
        float r0 = 0.f, r1 = 0.f, r2 = 0.f;
        for (int wv = 0; wv < nwaves; ++wv) {
          r0 += s_rb[wv][tid][0];
          r1 += s_rb[wv][tid][1];
          r2 += s_rb[wv][tid][2];
        }
        float* dst = a.rbar + 3 * static_cast<int64_t>(s_sl[tid]);
        if (a.rbar_accumulate) {
          dst[0] += r0;
          dst[1] += r1;
          dst[2] += r2;
        } else {
          dst[0] = r0;
          dst[1] = r1;
          dst[2] = r2;
        }
      }
      __syncthreads();
    }
  }
  // combine the edge slots of the wave (different edges of the same sender)
  for (int off = cp; off < kWave; off <<= 1)
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) {
        if constexpr (NEED_P) P[q][mi] += __shfl_xor(P[q][mi], off);
        if constexpr (TAN) Pd[q][mi] += __shfl_xor(Pd[q][mi], off);
      }
  if (slot == 0 && wvalid) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (q < a.g.nb)
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) {
          const int64_t o = (row0 + mi) * a.ld_state + a.state_col0 + static_cast<int64_t>(q) * a.c_out + w;
          if constexpr (NEED_P) a.P[o] = P[q][mi];
          if constexpr (TAN) a.Pdot[o] = Pd[q][mi];
        }
  }
}

template <int LI, int LO, int NBQ, bool TAN>
__global__ __launch_bounds__(256) void bwd_uvu_kernel(const BwdUvuArgs a) {
  constexpr int NI = 2 * LI + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  constexpr bool POS = !TAN;   // position adjoint only in the first-order pass
  using L = BwdLds<NB, NI, NO, true, TAN>;
  __shared__ float s_edge[64 * L::kStride];
  __shared__ int s_i[64];
  __shared__ int s_sl[64];
  __shared__ float s_rb[kMaxTiles][64][3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  const int u = wave * cp + (lane - slot * cp);
  const bool uvalid = u < a.c;
  const bool want_pos = POS && a.rbar != nullptr;
  float wv[NB], wbar[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    wv[q] = (uvalid && q < a.g.nb) ? a.w[q * a.c + u] : 0.f;
    wbar[q] = 0.f;
  }
  for (int j = blockIdx.x; j < a.n_nodes; j += gridDim.x) {
    float xj[NI], xb[NI];
    const float* xr = a.x + static_cast<int64_t>(j) * a.x_dim + a.xoff + u;
#pragma unroll
    for (int mi = 0; mi < NI; ++mi) {
      xj[mi] = uvalid ? xr[mi * a.c] : 0.f;
      xb[mi] = 0.f;
    }
    const int k0 = a.s_rowptr[j], k1 = a.s_rowptr[j + 1];
    for (int base = k0; base < k1; base += kWave) {
      const int ne = min(kWave, k1 - base);
      if (tid < ne) {
        const int i = a.s_col[base + tid];
        bwd_fill_edge<NB, NI, NO, true, TAN>(a.g, a.cg, a.ls, a.pos, a.pos_dot, j, i, s_edge + tid * L::kStride);
        s_i[tid] = i;
        s_sl[tid] = a.s_slot[base + tid];
      }
      __syncthreads();
      const int trips = (ne + nslots - 1) / nslots;
      for (int it = 0; it < trips; ++it) {
        const int t = it * nslots + slot;
        const bool tvalid = t < ne;
        const float* e = s_edge + (tvalid ? t : 0) * L::kStride;
        float zb[NO];
        const float* zr = a.z_bar + static_cast<int64_t>(tvalid ? s_i[t] : 0) * a.z_dim + a.zoff + u;
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) zb[mo] = (tvalid && uvalid) ? zr[mo * a.c] : 0.f;
        float Q[NI], Qd[NI];
        float h = 0.f, hd = 0.f;
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) {
          float s = 0.f, sd = 0.f;
#pragma unroll
          for (int mo = 0; mo < NO; ++mo) {
            s += e[L::kCy + mi * NO + mo] * zb[mo];
            if constexpr (TAN) sd += e[L::kCyDot + mi * NO + mo] * zb[mo];
          }
          Q[mi] = s;
          Qd[mi] = sd;
          h += xj[mi] * s;
          hd += xj[mi] * sd;
        }
        float we = 0.f, wed = 0.f, wdr = 0.f;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          we += e[L::kPhi + q] * wv[q];
          if constexpr (TAN) wed += e[L::kPhiDot + q] * wv[q];
          wdr += e[L::kDphi + q] * wv[q];
        }
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) xb[mi] += TAN ? (wed * Q[mi] + we * Qd[mi]) : we * Q[mi];
#pragma unroll
        for (int q = 0; q < NB; ++q)
          wbar[q] += TAN ? (e[L::kPhiDot + q] * h + e[L::kPhi + q] * hd) : e[L::kPhi + q] * h;
        if (want_pos) {
          const float srad = wdr * h;
          float rb[3];
#pragma unroll
          for (int d = 0; d < 3; ++d) {
            float s = 0.f;
#pragma unroll
            for (int mi = 0; mi < NI; ++mi) {
              float zc = 0.f;
#pragma unroll
              for (int mo = 0; mo < NO; ++mo) zc += e[L::kCdy + d * L::CY + mi * NO + mo] * zb[mo];
              s += xj[mi] * zc;
            }
            rb[d] = slot_sum(srad * e[L::kU + d] + we * s, cp);
          }
          if (tvalid && lane == slot * cp) {
            s_rb[wave][t][0] = rb[0];
            s_rb[wave][t][1] = rb[1];
            s_rb[wave][t][2] = rb[2];
          }
        }
      }
      __syncthreads();
      if (want_pos) {
        if (tid < ne) {
          float r0 = 0.f, r1 = 0.f, r2 = 0.f;
          for (int w2 = 0; w2 < nwaves; ++w2) {
            r0 += s_rb[w2][tid][0];
            r1 += s_rb[w2][tid][1];
            r2 += s_rb[w2][tid][2];
          }
          float* dst = a.rbar + 3 * static_cast<int64_t>(s_sl[tid]);
          if (a.rbar_accumulate) {
            dst[0] += r0;
            dst[1] += r1;
            dst[2] += r2;
          } else {
            dst[0] = r0;
            dst[1] = r1;
            dst[2] = r2;
          }
        }
        __syncthreads();
      }
    }
    for (int off = cp; off < kWave; off <<= 1)
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) xb[mi] += __shfl_xor(xb[mi], off);
    if (a.x_bar && slot == 0 && uvalid) {
      float* xo = a.x_bar + static_cast<int64_t>(j) * a.x_dim + a.xoff + u;
#pragma unroll
      for (int mi = 0; mi < NI; ++mi) {
        if (a.xbar_accumulate)
          xo[mi * a.c] += xb[mi];
        else
          xo[mi * a.c] = xb[mi];
      }
    }
  }
  for (int off = cp; off < kWave; off <<= 1)
#pragma unroll
    for (int q = 0; q < NB; ++q) wbar[q] += __shfl_xor(wbar[q], off);
  if (a.wbar_part && slot == 0 && uvalid) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (q < a.g.nb) a.wbar_part[(static_cast<int64_t>(blockIdx.x) * a.g.nb + q) * a.c + u] = wbar[q];
  }
}

template <int LI, int LO, bool NEED_P, bool POS, bool TAN>
hipError_t bwd_uvw_nb(const BwdUvwArgs& a, int nsend, int ntiles, hipStream_t s) {
  dim3 grid(nsend), block(64 * ntiles);
  switch ((a.g.nb + 3) / 4) {
    case 1: hipLaunchKernelGGL((bwd_uvw_kernel<LI, LO, 1, NEED_P, POS, TAN>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((bwd_uvw_kernel<LI, LO, 2, NEED_P, POS, TAN>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((bwd_uvw_kernel<LI, LO, 3, NEED_P, POS, TAN>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_uvw_kernel<LI, LO, 4, NEED_P, POS, TAN>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int LI, int LO, bool TAN>
hipError_t bwd_uvu_nb(const BwdUvuArgs& a, int nblocks, int ntiles, hipStream_t s) {
  dim3 grid(nblocks), block(64 * ntiles);
  switch ((a.g.nb + 3) / 4) {
    case 1: hipLaunchKernelGGL((bwd_uvu_kernel<LI, LO, 1, TAN>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((bwd_uvu_kernel<LI, LO, 2, TAN>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((bwd_uvu_kernel<LI, LO, 3, TAN>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_uvu_kernel<LI, LO, 4, TAN>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

#define ETPC_LL_DISPATCH(CALL)                 \
  switch (li * 4 + lo) {                       \
    case 0: return CALL(0, 0);                 \
    case 1: return CALL(0, 1);                 \
    case 2: return CALL(0, 2);                 \
    case 3: return CALL(0, 3);                 \
    case 4: return CALL(1, 0);                 \
    case 5: return CALL(1, 1);                 \
    case 6: return CALL(1, 2);                 \
    case 7: return CALL(1, 3);                 \
    case 8: return CALL(2, 0);                 \
    case 9: return CALL(2, 1);                 \
    case 10: return CALL(2, 2);                \
    case 11: return CALL(2, 3);                \
    case 12: return CALL(3, 0);                \
    case 13: return CALL(3, 1);                \
    case 14: return CALL(3, 2);                \
    default: return CALL(3, 3);                \
  }

template <bool NEED_P, bool POS, bool TAN>
hipError_t launch_bwd_uvw_t(const BwdUvwArgs& a, int li, int lo, int nsend, int ntiles, hipStream_t s) {
#define ETPC_CALL(LI, LO) bwd_uvw_nb<LI, LO, NEED_P, POS, TAN>(a, nsend, ntiles, s)
  ETPC_LL_DISPATCH(ETPC_CALL)
#undef ETPC_CALL
}

template <bool TAN>
hipError_t launch_bwd_uvu_t(const BwdUvuArgs& a, int li, int lo, int nblocks, int ntiles, hipStream_t s) {
#define ETPC_CALL(LI, LO) bwd_uvu_nb<LI, LO, TAN>(a, nblocks, ntiles, s)
  ETPC_LL_DISPATCH(ETPC_CALL)
#undef ETPC_CALL
}

}  // namespace bwd_detail
}  // namespace etpc
