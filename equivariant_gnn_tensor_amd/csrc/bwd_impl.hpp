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
#include "wave.hpp"
#include "cg_tables.inc"
#include "triples.hpp"

namespace etpc {
namespace bwd_detail {

constexpr int kMaxTiles = 4;

// z_bar gathers kept in flight per edge slot in the sender traversals
#ifndef ETPC_BWD_PREFETCH
#define ETPC_BWD_PREFETCH 2
#endif
constexpr int kPrefetch = ETPC_BWD_PREFETCH;
// The radial contractions of the position adjoint, T = sum_q phi_q Xt[q] and
// G = sum_q phi'_q Xt[q], on the matrix cores (1) or on the VALU (0).
#ifndef ETPC_BWD_XT_MFMA
#define ETPC_BWD_XT_MFMA 1
#endif
constexpr bool kXtMfma = ETPC_BWD_XT_MFMA != 0;
static_assert(!kXtMfma || kPrefetch % 2 == 0, "the matrix-core radial contraction covers two trips");

// What may cross the scheduling barrier placed after each pipelined gather: LDS reads and
// writes (0x80 | 0x100 | 0x200), so record reads can be hoisted; global loads never.
constexpr int kSchedMask = 0x380;

// First-order uvu backward: the register-budgeted kernel with matrix-core radial weights
// and W_bar partials (1) or the general uvu sender traversal (0).
#ifndef ETPC_BWD_UVU_FIRST
#define ETPC_BWD_UVU_FIRST 1
#endif
constexpr bool kUvuFirst = ETPC_BWD_UVU_FIRST != 0;
// z_bar gathers in flight per edge slot in the first-order uvu traversal (even; 4 and 6
// measured 3-7% slower: more registers, no more bandwidth)
#ifndef ETPC_BWD_UVU_PREFETCH
#define ETPC_BWD_UVU_PREFETCH 2
#endif
constexpr int kUvuPrefetch = ETPC_BWD_UVU_PREFETCH;
// Register budget of the first-order uvu traversal as resident waves per SIMD (0: the
// compiler's choice, 2 waves for most paths).  Three waves (168 VGPRs, 0-28 bytes per lane
// spilled, 48-64 for l_in = l_sh = 3) is what the workgroup's LDS allows; with a persistent
// grid of 4608 workgroups it measured 28% faster than the compiler's choice on the
// channelwise workload (backward traversals 16.4 -> 11.8 ms per step).
#ifndef ETPC_BWD_UVU_WAVES
#define ETPC_BWD_UVU_WAVES 3
#endif
#if ETPC_BWD_UVU_WAVES > 0
#define ETPC_BWD_UVU_ATTR __attribute__((amdgpu_waves_per_eu(ETPC_BWD_UVU_WAVES)))
#else
#define ETPC_BWD_UVU_ATTR
#endif

// Edge slots of the sender traversals are at least 16 lanes wide (the host rounds the
// channel count up), so a per-edge lane sum is a DPP row sum per 16 lanes (no branch, no
// LDS round trip) plus a sum over the cp/16 rows of the slot, done through LDS.
__device__ inline int rows_per_slot(int cp) { return cp / 16; }

typedef float f4v __attribute__((ext_vector_type(4)));

// Compact per-edge record for the sender traversals (LDS, one per edge of a chunk):
// phi[NB], phi'[NB] (positions), dphi[NB] along pos_dot (tangent), phi''[NB] (Hessian),
// Y[NS], dY/dr[3][NS] (positions), dY[NS] along pos_dot (tangent, Hessian),
// d(dY/dr)[3][NS] along pos_dot (Hessian), u[3] (positions), du[3] and d|r| along
// pos_dot (Hessian).  The coupling tensor is not stored per edge: its compile-time
// sparse form is applied per lane (CgTab).
// Field offsets are rounded up to multiples of A floats.  A = 4 puts every field on a
// 16-byte boundary, so its broadcast reads are ds_read_b128: the uvu traversal gains from
// that (-2%), while the uvw traversals measured slower with the larger record (+4%), so
// they keep the packed one (A = 1).
template <int A>
constexpr int rec_align(int n) { return (n + A - 1) / A * A; }
template <int NB, int NS, bool POS, bool TAN, bool HESS = false, int A = 1>
struct BwdRec {
  static constexpr int kNSP = rec_align<A>(NS);   // row length of the dY/dr and d(dY/dr) rows
  static constexpr int kPhi = 0;
  static constexpr int kDphi = rec_align<A>(NB);
  static constexpr int kPhiDot = rec_align<A>(kDphi + (POS ? NB : 0));
  static constexpr int kDDphi = rec_align<A>(kPhiDot + (TAN ? NB : 0));
  static constexpr int kY = rec_align<A>(kDDphi + (HESS ? NB : 0));
  static constexpr int kDY = rec_align<A>(kY + NS);
  static constexpr int kYDot = rec_align<A>(kDY + (POS ? 3 * kNSP : 0));
  static constexpr int kDDY = rec_align<A>(kYDot + ((TAN || HESS) ? NS : 0));
  static constexpr int kU = rec_align<A>(kDDY + (HESS ? 3 * kNSP : 0));
  static constexpr int kUDot = kU + (POS ? 3 : 0);
  static constexpr int kRhoDot = kUDot + (HESS ? 3 : 0);
  static constexpr int kStride = rec_align<A>(kRhoDot + (HESS ? 1 : 0) + 1);
};

template <int LS, int NB, bool POS, bool TAN, bool NEED_D, bool HESS = false, int A = 1>
__device__ inline void bwd_fill_rec(const GeomParams& g, const float* __restrict__ pos,
                                    const float* __restrict__ pos_dot, int j, int i, float* __restrict__ e) {
  constexpr int NS = 2 * LS + 1;
  using R = BwdRec<NB, NS, POS, TAN, HESS, A>;
  float rx, ry, rz;
  edge_vector(g, pos, j, i, rx, ry, rz);
  const float r = sqrtf(rx * rx + ry * ry + rz * rz);
  const float ir = 1.f / r;
  const float ux = rx * ir, uy = ry * ir, uz = rz * ir;
  float phi[NB], dphi[NB], ddphi[NB];
  radial_eval<NB>(g, r, phi, NEED_D ? dphi : nullptr, HESS ? ddphi : nullptr);
  float y[7];
  sh_eval(LS, ux, uy, uz, y);
  float gy[7][3];
  if constexpr (POS || TAN) sh_grad_r(LS, ux, uy, uz, ir, y, gy);
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    e[R::kPhi + q] = phi[q];
    if constexpr (POS) e[R::kDphi + q] = dphi[q];
    if constexpr (HESS) e[R::kDDphi + q] = ddphi[q];
  }
#pragma unroll
  for (int m = 0; m < NS; ++m) {
    e[R::kY + m] = y[m];
    if constexpr (POS) {
      e[R::kDY + m] = gy[m][0];
      e[R::kDY + R::kNSP + m] = gy[m][1];
      e[R::kDY + 2 * R::kNSP + m] = gy[m][2];
    }
  }
  if constexpr (TAN || HESS) {
    // edge-vector tangent r_dot = pos_dot_sender - pos_dot_receiver (Eq. 8 differentiated)
    const float dx = pos_dot[3 * j + 0] - pos_dot[3 * i + 0];
    const float dy = pos_dot[3 * j + 1] - pos_dot[3 * i + 1];
    const float dz = pos_dot[3 * j + 2] - pos_dot[3 * i + 2];
    const float rdot = ux * dx + uy * dy + uz * dz;
    if constexpr (TAN) {
#pragma unroll
      for (int q = 0; q < NB; ++q) e[R::kPhiDot + q] = dphi[q] * rdot;
    }
#pragma unroll
    for (int m = 0; m < NS; ++m) e[R::kYDot + m] = gy[m][0] * dx + gy[m][1] * dy + gy[m][2] * dz;
    if constexpr (HESS) {
      const float udx = (dx - ux * rdot) * ir, udy = (dy - uy * rdot) * ir, udz = (dz - uz * rdot) * ir;
      float ddy[7][3];
      sh_grad_r_dir(LS, ux, uy, uz, ir, y, gy, udx, udy, udz, rdot, ddy);
#pragma unroll
      for (int m = 0; m < NS; ++m) {
        e[R::kDDY + m] = ddy[m][0];
        e[R::kDDY + R::kNSP + m] = ddy[m][1];
        e[R::kDDY + 2 * R::kNSP + m] = ddy[m][2];
      }
      e[R::kUDot + 0] = udx;
      e[R::kUDot + 1] = udy;
      e[R::kUDot + 2] = udz;
      e[R::kRhoDot] = rdot;
    }
  }
  if constexpr (POS) {
    e[R::kU + 0] = ux;
    e[R::kU + 1] = uy;
    e[R::kU + 2] = uz;
  }
}

// V[m_in][m_sh] = sum_m_out c[m_in][m_sh][m_out] zb[m_out] with the compile-time sparse table
template <int LI, int LS, int LO>
__device__ inline void cg_contract_out(const float* __restrict__ zb, float (*__restrict__ V)[2 * LS + 1]) {
  using C = CgTab<LI, LS, LO>;
#pragma unroll
  for (int a = 0; a < 2 * LI + 1; ++a)
#pragma unroll
    for (int b = 0; b < 2 * LS + 1; ++b) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 2 * LO + 1; ++m)
        if (C::v[a][b][m] != 0.f) s += C::v[a][b][m] * zb[m];
      V[a][b] = s;
    }
}

// Sender traversal for one uvw path (compile-time l_in, l_sh, l_out).  With HESS (and
// POS) the per-edge output is not r_bar_e but its directional derivative along
// r_dot_e = pos_dot_sender - pos_dot_receiver, i.e. H_e r_dot_e with H_e the Hessian of the
// edge's term of <z_bar, z> in the edge vector: the position term of double backward.
// SPLIT: a.nparts waves per channel tile share the sender's edges (small launches);
// without it the part count is the constant 1 and that code folds away.
template <int LI, int LS, int LO, int NBQ, bool NEED_P, bool POS, bool TAN, bool HESS = false, bool SPLIT = false>
__global__ __launch_bounds__(256) void bwd_uvw_kernel(const BwdUvwArgs a) {
  constexpr int NI = 2 * LI + 1, NS = 2 * LS + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  static_assert(!HESS || (POS && !TAN && !NEED_P), "the Hessian pass is a position-only pass");
  using R = BwdRec<NB, NS, POS, TAN, HESS>;
  __shared__ __attribute__((aligned(16))) float s_edge[64 * R::kStride];
  __shared__ int s_i[64];
  __shared__ int s_sl[64];
  // [nwaves][64][rows][3] edge-adjoint partials, then (nparts > 1) the state exchange
  extern __shared__ float s_dyn[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  // Senders in decreasing degree when an order is given: the hardware hands out
  // workgroups in index order, so the last ones to start are the short ones and the
  // launch ends with a short tail.  Each sender keeps its own state rows, so the
  // results do not depend on the order.
  const int j = a.order ? a.order[blockIdx.x] : a.send0 + static_cast<int>(blockIdx.x);
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  // waves are (part, tile): tile = channel range, part = share of the sender's edges
  const int nparts = SPLIT ? a.nparts : 1;
  const int ntiles = nwaves / nparts;
  const int tile = SPLIT ? wave % ntiles : wave, part = SPLIT ? wave / ntiles : 0;
  const int tslots = nslots * nparts;     // edge slots of the workgroup per trip
  const int gslot = part * nslots + slot;
  const int w = tile * cp + (lane - slot * cp);
  const bool wvalid = w < a.c_out;
  const int rows = rows_per_slot(cp);
  const int row_in_slot = (lane - slot * cp) >> 4;
  const bool row_leader = (lane & 15) == 0;
  const int q4 = lane & 3;
  const int64_t row0 = static_cast<int64_t>(j - a.send0) * NI;
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
  f4v P[NI][NBQ], Pd[NI][NBQ];
#pragma unroll
  for (int mi = 0; mi < NI; ++mi)
#pragma unroll
    for (int qq = 0; qq < NBQ; ++qq) {
      P[mi][qq] = f4v{0.f, 0.f, 0.f, 0.f};
      Pd[mi][qq] = f4v{0.f, 0.f, 0.f, 0.f};
    }
  const int k0 = a.s_rowptr[j], k1 = a.s_rowptr[j + 1];
  for (int base = k0; base < k1; base += kWave) {
    const int ne = min(kWave, k1 - base);
    if (tid < ne) {
      const int i = a.s_col[base + tid];
      bwd_fill_rec<LS, NB, POS, TAN, POS || TAN, HESS>(a.g, a.pos, a.pos_dot, j, i, s_edge + tid * R::kStride);
      s_i[tid] = i;
      s_sl[tid] = a.s_slot[base + tid];
    }
    __syncthreads();
    const int trips = (ne + tslots - 1) / tslots;
    // z_bar rows of the next kPrefetch edges of this slot are in flight while one is used
    float zq[kPrefetch][NO];
    // Unconditional loads from a clamped in-bounds address (no branch per load); lanes
    // without an edge are zeroed when the row is consumed, not here, so nothing waits
    // on the load before its own trip.
    // receiver of trip slot t (0 past the chunk: a clamped, harmless row)
    auto recv_of = [&](int t) { return t < ne ? s_i[t] : 0; };
    auto gather = [&](int i, float* dst) {
      const float* zr = a.z_bar + static_cast<int64_t>(i) * a.z_dim + a.zoff + (wvalid ? w : 0);
#pragma unroll
      for (int mo = 0; mo < NO; ++mo) dst[mo] = zr[mo * a.c_out];
    };
    // the receiver index of each gather is read one round ahead, so forming the gather
    // address never waits on an LDS read
    int next_i[kPrefetch];
#pragma unroll
    for (int pf = 0; pf < kPrefetch; ++pf) {
      gather(recv_of(pf * tslots + gslot), zq[pf]);
      next_i[pf] = recv_of((pf + kPrefetch) * tslots + gslot);
      // Pass the first rows through an arithmetic op: when every value entering the
      // loop-carried registers is a plain load, the optimizer merges them into one load
      // at the top of the loop, which undoes the prefetch.
#pragma unroll
      for (int mo = 0; mo < NO; ++mo) zq[pf][mo] += 0.f;
    }
    for (int it0 = 0; it0 < trips; it0 += kPrefetch) {
      f4v TG[NI];
#pragma unroll
      for (int pf = 0; pf < kPrefetch; ++pf) {
        // Position adjoint, radial contractions of two trips at once: with 4x4x1
        // matrix-core blocks of four lanes, row r of a block takes phi (r = 0, 1) or
        // phi' (r = 2, 3) of the edge of trip it0 + pf + (r & 1), and each lane's column is
        // its own Xt[q][m_in]; so after the NB accumulations register r of a lane holds T
        // (r < 2) or G (r >= 2) of that edge for the lane's channel.  A padding trip reads
        // edge 0's record; its results feed only the edge adjoint that is never stored.
        if constexpr (POS && kXtMfma) {
          if (pf % 2 == 0) {
            const int r4 = lane & 3;
            const int tt = (it0 + pf + (r4 & 1)) * tslots + gslot;
            const float* er = s_edge + (tt < ne ? tt : 0) * R::kStride + (r4 < 2 ? R::kPhi : R::kDphi);
#pragma unroll
            for (int mi = 0; mi < NI; ++mi) TG[mi] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NB; ++q) {
              const float aq = er[q];
#pragma unroll
              for (int mi = 0; mi < NI; ++mi)
                TG[mi] = __builtin_amdgcn_mfma_f32_4x4x1f32(aq, xt[q][mi], TG[mi], 0, 0, 0);
            }
          }
        }
        // trips run in whole groups of kPrefetch (no exit inside the unrolled body, which
        // would make the compiler copy the loop-carried registers and wait on the loads);
        // a padding trip has t >= ne, gathers zeros and adds exact zeros
        const int it = it0 + pf;
        const int t = it * tslots + gslot;
        const bool tvalid = t < ne;
        const float* e = s_edge + (tvalid ? t : 0) * R::kStride;
        // No mask on the gathered row: a padding trip reads real data (edge 0's record and a
        // clamped row), so only its state update is masked (through phi below), its edge
        // adjoint is never stored, and lanes past c_out hold Xt = 0, so they add zeros
        // to every lane sum.
        float zb[NO];
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) zb[mo] = zq[pf][mo];
        float V[NI][NS];
        cg_contract_out<LI, LS, LO>(zb, V);
        // the row is consumed: its registers take the gather kPrefetch trips ahead (no
        // register copy, so nothing waits for that load until its own trip); the
        // scheduling barrier keeps the loads here instead of sunk to the loop end
        gather(next_i[pf], zq[pf]);
        next_i[pf] = recv_of(t + 2 * kPrefetch * tslots);
        __builtin_amdgcn_sched_barrier(kSchedMask);
        float Q[NI], Qd[NI];
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) {
          float s = 0.f, sd = 0.f;
#pragma unroll
          for (int my = 0; my < NS; ++my) {
            s += e[R::kY + my] * V[mi][my];
            if constexpr (TAN || HESS) sd += e[R::kYDot + my] * V[mi][my];
          }
          Q[mi] = s;
          Qd[mi] = sd;
        }
#pragma unroll
        for (int qq = 0; qq < NBQ; ++qq) {
          const float ph = tvalid ? e[R::kPhi + 4 * qq + q4] : 0.f;
          if constexpr (NEED_P) {
#pragma unroll
            for (int mi = 0; mi < NI; ++mi)
              P[mi][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(ph, Q[mi], P[mi][qq], 0, 0, 0);
          }
          if constexpr (TAN) {
            const float phd = tvalid ? e[R::kPhiDot + 4 * qq + q4] : 0.f;
#pragma unroll
            for (int mi = 0; mi < NI; ++mi) {
              Pd[mi][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(phd, Q[mi], Pd[mi][qq], 0, 0, 0);
              Pd[mi][qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(ph, Qd[mi], Pd[mi][qq], 0, 0, 0);
            }
          }
        }
        if constexpr (POS) {
          // radial part: sum_q phi'_q phi_bar_q = sum_m_in G[m_in] Q[m_in], G = sum_q phi'_q Xt[q];
          // angular part: sum_m_sh dY[d][m_sh] Wy[m_sh], Wy = sum_m_in T[m_in] V[m_in][m_sh], T = sum_q phi_q Xt[q]
          float srad = 0.f, sradd = 0.f;
          float wy[NS], wg[NS];
#pragma unroll
          for (int my = 0; my < NS; ++my) wy[my] = wg[my] = 0.f;
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) {
            float tq = 0.f, gq = 0.f, g2 = 0.f;
            if constexpr (kXtMfma) {
              tq = TG[mi][pf & 1];
              gq = TG[mi][2 + (pf & 1)];
            } else {
#pragma unroll
              for (int q = 0; q < NB; ++q) {
                tq += e[R::kPhi + q] * xt[q][mi];
                gq += e[R::kDphi + q] * xt[q][mi];
              }
            }
            if constexpr (HESS) {
#pragma unroll
              for (int q = 0; q < NB; ++q) g2 += e[R::kDDphi + q] * xt[q][mi];
            }
            srad += gq * Q[mi];
            // Hessian pass: d srad = sum (rho_dot G2 Q + G dQ), dQ = dY . V
            if constexpr (HESS) sradd += e[R::kRhoDot] * g2 * Q[mi] + gq * Qd[mi];
#pragma unroll
            for (int my = 0; my < NS; ++my) {
              wy[my] += tq * V[mi][my];
              if constexpr (HESS) wg[my] += gq * V[mi][my];   // dT = rho_dot G, so dWy = rho_dot Wg
            }
          }
          float rb[3];
#pragma unroll
          for (int d = 0; d < 3; ++d) {
            float s = 0.f;
#pragma unroll
            for (int my = 0; my < NS; ++my) {
              if constexpr (HESS)
                s += e[R::kDDY + d * R::kNSP + my] * wy[my] + e[R::kRhoDot] * e[R::kDY + d * R::kNSP + my] * wg[my];
              else
                s += e[R::kDY + d * R::kNSP + my] * wy[my];
            }
            rb[d] = s;
          }
          float* sr = s_dyn + ((wave * 64 + (tvalid ? t : 0)) * rows + row_in_slot) * 3;
          float lanev[3];
#pragma unroll
          for (int d = 0; d < 3; ++d) {
            // r_bar = srad u + dY^T Wy; its tangent = d srad u + srad du + d(dY)^T Wy + dY^T dWy
            lanev[d] = HESS ? sradd * e[R::kU + d] + srad * e[R::kUDot + d] + rb[d] : srad * e[R::kU + d] + rb[d];
          }
          row_sum16x3(lanev[0], lanev[1], lanev[2]);
          if (tvalid && row_leader) {
            sr[0] = lanev[0];
            sr[1] = lanev[1];
            sr[2] = lanev[2];
          }
        }
      }
    }
    __syncthreads();
    if constexpr (POS) {
      if (tid < ne) {
        // the waves of every channel tile of the part that took this edge
        const int pe = (tid % tslots) / nslots;
        float r0 = 0.f, r1 = 0.f, r2 = 0.f;
        for (int tl = 0; tl < ntiles; ++tl)
          for (int r = 0; r < rows; ++r) {
            const int w2 = pe * ntiles + tl;
            const float* src = s_dyn + ((w2 * 64 + tid) * rows + r) * 3;
            r0 += src[0];
            r1 += src[1];
            r2 += src[2];
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
    for (int mi = 0; mi < NI; ++mi)
#pragma unroll
      for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (NEED_P) P[mi][qq][r] += __shfl_xor(P[mi][qq][r], off);
          if constexpr (TAN) Pd[mi][qq][r] += __shfl_xor(Pd[mi][qq][r], off);
        }
  if constexpr (NEED_P || TAN) {
    // parts 1.. hand their state to part 0 through LDS, one part at a time (fixed order)
    constexpr int kState = NI * NB * ((NEED_P ? 1 : 0) + (TAN ? 1 : 0));
    float* s_x = s_dyn + (POS ? nwaves * 64 * rows * 3 : 0) + (tile * 64 + lane) * kState;
    for (int pp = 1; pp < nparts; ++pp) {
      __syncthreads();
      if (part == pp && slot == 0) {
        int o = 0;
#pragma unroll
        for (int mi = 0; mi < NI; ++mi)
#pragma unroll
          for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if constexpr (NEED_P) s_x[o++] = P[mi][qq][r];
              if constexpr (TAN) s_x[o++] = Pd[mi][qq][r];
            }
      }
      __syncthreads();
      if (part == 0 && slot == 0) {
        int o = 0;
#pragma unroll
        for (int mi = 0; mi < NI; ++mi)
#pragma unroll
          for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if constexpr (NEED_P) P[mi][qq][r] += s_x[o++];
              if constexpr (TAN) Pd[mi][qq][r] += s_x[o++];
            }
      }
    }
  }
  if (part == 0 && slot == 0 && wvalid) {
#pragma unroll
    for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * qq + r < a.g.nb)
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) {
            const int64_t o =
                (row0 + mi) * a.ld_state + a.state_col0 + static_cast<int64_t>(4 * qq + r) * a.c_out + w;
            if constexpr (NEED_P) a.P[o] = P[mi][qq][r];
            if constexpr (TAN) a.Pdot[o] = Pd[mi][qq][r];
          }
  }
}

// With HESS the per-edge output is the tangent of r_bar_e along r_dot_e (the position
// term of double backward, as in the uvw traversal); x_bar and W_bar are not formed.
template <int LI, int LS, int LO, int NBQ, bool TAN, bool HESS = false>
__global__ __launch_bounds__(256) void bwd_uvu_kernel(const BwdUvuArgs a) {
  constexpr int NI = 2 * LI + 1, NS = 2 * LS + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  constexpr bool POS = !TAN;   // position adjoint only in the first-order and Hessian passes
  static_assert(!(HESS && TAN), "the Hessian pass has no tangent state");
  constexpr int kRecAlign = 4;
  using R = BwdRec<NB, NS, true, TAN, HESS, kRecAlign>;
  __shared__ __attribute__((aligned(16))) float s_edge[64 * R::kStride];
  __shared__ int s_i[64];
  __shared__ int s_sl[64];
  extern __shared__ float s_dyn[];   // [nwaves][64][rows][3]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  const int u = wave * cp + (lane - slot * cp);
  const bool uvalid = u < a.c;
  const int rows = rows_per_slot(cp);
  const int row_in_slot = (lane - slot * cp) >> 4;
  const bool row_leader = (lane & 15) == 0;
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
        bwd_fill_rec<LS, NB, true, TAN, true, HESS, kRecAlign>(a.g, a.pos, a.pos_dot, j, i,
                                                                s_edge + tid * R::kStride);
        s_i[tid] = i;
        s_sl[tid] = a.s_slot[base + tid];
      }
      __syncthreads();
      const int trips = (ne + nslots - 1) / nslots;
      // same software pipeline as the uvw sender traversal
      float zq[kPrefetch][NO];
      // (reading the receiver index one round ahead, as the uvw traversal does, measured
      // 2% slower here)
      auto gather = [&](int t, float* dst) {
        const int i = s_i[t < ne ? t : 0];
        const float* zr = a.z_bar + static_cast<int64_t>(t < ne ? i : 0) * a.z_dim + a.zoff + (uvalid ? u : 0);
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) dst[mo] = zr[mo * a.c];
      };
#pragma unroll
      for (int pf = 0; pf < kPrefetch; ++pf) {
        gather(pf * nslots + slot, zq[pf]);
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) zq[pf][mo] += 0.f;   // not a plain load
      }
      for (int it0 = 0; it0 < trips; it0 += kPrefetch) {
#pragma unroll
        for (int pf = 0; pf < kPrefetch; ++pf) {
          const int t = (it0 + pf) * nslots + slot;
          const bool tvalid = t < ne;
          const float* e = s_edge + (tvalid ? t : 0) * R::kStride;
          float zb[NO];
#pragma unroll
          for (int mo = 0; mo < NO; ++mo) zb[mo] = zq[pf][mo];   // masked below, through w_e and h
          gather(t + kPrefetch * nslots, zq[pf]);
          __builtin_amdgcn_sched_barrier(kSchedMask);
          float V[NI][NS];
          cg_contract_out<LI, LS, LO>(zb, V);
          float Q[NI], Qd[NI];
          float h = 0.f, hd = 0.f;
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) {
            float s = 0.f, sd = 0.f;
#pragma unroll
            for (int my = 0; my < NS; ++my) {
              s += e[R::kY + my] * V[mi][my];
              if constexpr (TAN || HESS) sd += e[R::kYDot + my] * V[mi][my];
            }
            Q[mi] = s;
            Qd[mi] = sd;
            h += xj[mi] * s;
            hd += xj[mi] * sd;
          }
          float we = 0.f, wed = 0.f, wdr = 0.f, wdd = 0.f;
#pragma unroll
          for (int q = 0; q < NB; ++q) {
            we += e[R::kPhi + q] * wv[q];
            if constexpr (TAN) wed += e[R::kPhiDot + q] * wv[q];
            wdr += e[R::kDphi + q] * wv[q];
            if constexpr (HESS) wdd += e[R::kDDphi + q] * wv[q];
          }
          if constexpr (!HESS) {
            // a padding trip (real but foreign data) adds nothing; lanes past c hold
            // x = 0 and w = 0, so their h, w_e and lane-sum terms are zero already
            const float wem = tvalid ? we : 0.f, wedm = tvalid ? wed : 0.f;
            const float hm = tvalid ? h : 0.f, hdm = tvalid ? hd : 0.f;
#pragma unroll
            for (int mi = 0; mi < NI; ++mi) xb[mi] += TAN ? (wedm * Q[mi] + wem * Qd[mi]) : wem * Q[mi];
#pragma unroll
            for (int q = 0; q < NB; ++q)
              wbar[q] += TAN ? (e[R::kPhiDot + q] * hm + e[R::kPhi + q] * hdm) : e[R::kPhi + q] * hm;
          }
          if (want_pos) {
            const float srad = wdr * h;
            float wy[NS];
#pragma unroll
            for (int my = 0; my < NS; ++my) {
              float s = 0.f;
#pragma unroll
              for (int mi = 0; mi < NI; ++mi) s += xj[mi] * V[mi][my];
              wy[my] = s;
            }
            float rb[3], rbd[3];
#pragma unroll
            for (int d = 0; d < 3; ++d) {
              float s = 0.f, sd = 0.f;
#pragma unroll
              for (int my = 0; my < NS; ++my) {
                s += e[R::kDY + d * R::kNSP + my] * wy[my];
                if constexpr (HESS) sd += e[R::kDDY + d * R::kNSP + my] * wy[my];
              }
              rb[d] = s;
              rbd[d] = sd;
            }
            float* sr = s_dyn + ((wave * 64 + (tvalid ? t : 0)) * rows + row_in_slot) * 3;
            float lanev[3];
#pragma unroll
            for (int d = 0; d < 3; ++d) {
              // r_bar = srad u + w_e dY^T Wy (srad = w_e' h); its tangent along r_dot:
              // d srad u + srad du + d w_e dY^T Wy + w_e d(dY)^T Wy, with d w_e = rho_dot w_e',
              // d srad = rho_dot w_e'' h + w_e' dh
              if constexpr (HESS) {
                const float rho_dot = e[R::kRhoDot];
                const float sradd = rho_dot * wdd * h + wdr * hd;
                lanev[d] = sradd * e[R::kU + d] + srad * e[R::kUDot + d] + rho_dot * wdr * rb[d] + we * rbd[d];
              } else {
                lanev[d] = srad * e[R::kU + d] + we * rb[d];
              }
            }
            row_sum16x3(lanev[0], lanev[1], lanev[2]);
            if (tvalid && row_leader) {
              sr[0] = lanev[0];
              sr[1] = lanev[1];
              sr[2] = lanev[2];
            }
          }
        }
      }
      __syncthreads();
      if (want_pos) {
        if (tid < ne) {
          float r0 = 0.f, r1 = 0.f, r2 = 0.f;
          for (int w2 = 0; w2 < nwaves; ++w2)
            for (int r = 0; r < rows; ++r) {
              const float* src = s_dyn + ((w2 * 64 + tid) * rows + r) * 3;
              r0 += src[0];
              r1 += src[1];
              r2 += src[2];
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

// First-order uvu sender traversal (x_bar, W_bar partials, r_bar), the same per-edge
// arithmetic as bwd_uvu_kernel with two parts moved to 4x4x1 matrix-core blocks of four
// lanes: the radial weights w_e = sum_q phi_q W[q][u] and w_e' = sum_q phi'_q W[q][u] of two
// trips at once (row r of a block takes phi (r < 2) or phi' (r >= 2) of trip it0 + pf +
// (r & 1), each lane's column its own W[q][u]), and the W_bar partials sum_e phi_q h_e
// (rows phi[4qq + r], every lane its own h), which frees the 2B FMAs and B accumulations
// per edge of the VALU form.  Its register budget (ETPC_BWD_UVU_WAVES) sets the occupancy.
template <int LI, int LS, int LO, int NBQ>
__global__ __launch_bounds__(256) ETPC_BWD_UVU_ATTR void bwd_uvu_first_kernel(const BwdUvuArgs a) {
  constexpr int NI = 2 * LI + 1, NS = 2 * LS + 1, NO = 2 * LO + 1, NB = 4 * NBQ;
  static_assert(kUvuPrefetch % 2 == 0, "the radial weights cover two trips");
  constexpr int kRecAlign = 4;
  using R = BwdRec<NB, NS, true, false, false, kRecAlign>;
  __shared__ __attribute__((aligned(16))) float s_edge[64 * R::kStride];
  __shared__ int s_i[64];
  __shared__ int s_sl[64];
  extern __shared__ float s_dyn[];   // [nwaves][64][rows][3]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int cp = a.cp;
  const int nslots = kWave / cp;
  const int slot = lane / cp;
  const int u = wave * cp + (lane - slot * cp);
  const bool uvalid = u < a.c;
  const int rows = rows_per_slot(cp);
  const int row_in_slot = (lane - slot * cp) >> 4;
  const bool row_leader = (lane & 15) == 0;
  const int q4 = lane & 3;
  const bool want_pos = a.rbar != nullptr;
  float wv[NB];
  f4v wb[NBQ];   // W_bar partials: register r of wb[qq] holds q = 4 qq + r
#pragma unroll
  for (int q = 0; q < NB; ++q) wv[q] = (uvalid && q < a.g.nb) ? a.w[q * a.c + u] : 0.f;
#pragma unroll
  for (int qq = 0; qq < NBQ; ++qq) wb[qq] = f4v{0.f, 0.f, 0.f, 0.f};
  for (int j = blockIdx.x; j < a.n_nodes; j += gridDim.x) {
    float xj[NI];
    const float* xr = a.x + static_cast<int64_t>(j) * a.x_dim + a.xoff + u;
#pragma unroll
    for (int mi = 0; mi < NI; ++mi) xj[mi] = uvalid ? xr[mi * a.c] : 0.f;
    float xb[NI];
#pragma unroll
    for (int mi = 0; mi < NI; ++mi) xb[mi] = 0.f;
    const int k0 = a.s_rowptr[j], k1 = a.s_rowptr[j + 1];
    for (int base = k0; base < k1; base += kWave) {
      const int ne = min(kWave, k1 - base);
      if (tid < ne) {
        const int i = a.s_col[base + tid];
        bwd_fill_rec<LS, NB, true, false, true, false, kRecAlign>(a.g, a.pos, a.pos_dot, j, i,
                                                                  s_edge + tid * R::kStride);
        s_i[tid] = i;
        s_sl[tid] = a.s_slot[base + tid];
      }
      __syncthreads();
      const int trips = (ne + nslots - 1) / nslots;
      float zq[kUvuPrefetch][NO];
      auto gather = [&](int t, float* dst) {
        const int i = s_i[t < ne ? t : 0];
        const float* zr = a.z_bar + static_cast<int64_t>(t < ne ? i : 0) * a.z_dim + a.zoff + (uvalid ? u : 0);
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) dst[mo] = zr[mo * a.c];
      };
#pragma unroll
      for (int pf = 0; pf < kUvuPrefetch; ++pf) {
        gather(pf * nslots + slot, zq[pf]);
#pragma unroll
        for (int mo = 0; mo < NO; ++mo) zq[pf][mo] += 0.f;   // not a plain load
      }
      for (int it0 = 0; it0 < trips; it0 += kUvuPrefetch) {
        f4v WE;
#pragma unroll
        for (int pf = 0; pf < kUvuPrefetch; ++pf) {
          if (pf % 2 == 0) {
            // w_e and w_e' = sum_q phi'_q W[q][u] of trips it0 + pf and it0 + pf + 1: row r of a
            // block takes phi (r < 2) or phi' (r >= 2) of trip it0 + pf + (r & 1)
            const int tt = (it0 + pf + (q4 & 1)) * nslots + slot;
            const float* er = s_edge + (tt < ne ? tt : 0) * R::kStride + (q4 < 2 ? R::kPhi : R::kDphi);
            WE = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NB; ++q) WE = __builtin_amdgcn_mfma_f32_4x4x1f32(er[q], wv[q], WE, 0, 0, 0);
          }
          const float we = WE[pf & 1], wdr = WE[2 + (pf & 1)];
          const int t = (it0 + pf) * nslots + slot;
          const bool tvalid = t < ne;
          const float* e = s_edge + (tvalid ? t : 0) * R::kStride;
          float zb[NO];
#pragma unroll
          for (int mo = 0; mo < NO; ++mo) zb[mo] = zq[pf][mo];   // masked below, through w_e and h
          gather(t + kUvuPrefetch * nslots, zq[pf]);
          __builtin_amdgcn_sched_barrier(kSchedMask);
          // a padding trip (real but foreign data) adds nothing; lanes past c hold x = 0 and
          // W = 0, so their h, w_e and lane-sum terms are zero already
          const float wem = tvalid ? we : 0.f;
          float wy[NS];
          float h = 0.f;
          float V[NI][NS];
          cg_contract_out<LI, LS, LO>(zb, V);
#pragma unroll
          for (int mi = 0; mi < NI; ++mi) {
            float s = 0.f;
#pragma unroll
            for (int my = 0; my < NS; ++my) s += e[R::kY + my] * V[mi][my];
            h += xj[mi] * s;
            xb[mi] += wem * s;
          }
#pragma unroll
          for (int my = 0; my < NS; ++my) {
            float s = 0.f;
#pragma unroll
            for (int mi = 0; mi < NI; ++mi) s += xj[mi] * V[mi][my];
            wy[my] = s;
          }
          const float hm = tvalid ? h : 0.f;
#pragma unroll
          for (int qq = 0; qq < NBQ; ++qq)
            wb[qq] = __builtin_amdgcn_mfma_f32_4x4x1f32(e[R::kPhi + 4 * qq + q4], hm, wb[qq], 0, 0, 0);
          if (want_pos) {
            const float srad = wdr * h;
            float lanev[3];
#pragma unroll
            for (int d = 0; d < 3; ++d) {
              float s = 0.f;
#pragma unroll
              for (int my = 0; my < NS; ++my) s += e[R::kDY + d * R::kNSP + my] * wy[my];
              // r_bar = w_e' h u + w_e dY^T Ybar
              lanev[d] = srad * e[R::kU + d] + we * s;
            }
            row_sum16x3(lanev[0], lanev[1], lanev[2]);
            float* sr = s_dyn + ((wave * 64 + (tvalid ? t : 0)) * rows + row_in_slot) * 3;
            if (tvalid && row_leader) {
              sr[0] = lanev[0];
              sr[1] = lanev[1];
              sr[2] = lanev[2];
            }
          }
        }
      }
      __syncthreads();
      if (want_pos) {
        if (tid < ne) {
          float r0 = 0.f, r1 = 0.f, r2 = 0.f;
          for (int w2 = 0; w2 < nwaves; ++w2)
            for (int r = 0; r < rows; ++r) {
              const float* src = s_dyn + ((w2 * 64 + tid) * rows + r) * 3;
              r0 += src[0];
              r1 += src[1];
              r2 += src[2];
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
    for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
      for (int r = 0; r < 4; ++r) wb[qq][r] += __shfl_xor(wb[qq][r], off);
  if (a.wbar_part && slot == 0 && uvalid) {
#pragma unroll
    for (int qq = 0; qq < NBQ; ++qq)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = 4 * qq + r;
        if (q < a.g.nb) a.wbar_part[(static_cast<int64_t>(blockIdx.x) * a.g.nb + q) * a.c + u] = wb[qq][r];
      }
  }
}

template <int LI, int LS, int LO, bool NEED_P, bool POS, bool TAN, bool HESS>
hipError_t bwd_uvw_nb(const BwdUvwArgs& a, int nsend, int ntiles, hipStream_t s) {
  const int nwaves = ntiles * a.nparts;
  dim3 grid(nsend), block(64 * nwaves);
  const int rows = a.cp / 16;
  const int ni = 2 * LI + 1, nb = a.g.nb <= 8 ? 8 : 16;
  const size_t state = a.nparts > 1 ? static_cast<size_t>(ntiles) * 64 * ni * nb * ((NEED_P ? 1 : 0) + (TAN ? 1 : 0)) : 0;
  const size_t dyn = sizeof(float) * ((POS ? 64 * 3 * rows * nwaves : 0) + state);
  const bool split = a.nparts > 1;
  if (a.g.nb <= 8) {
    if (split)
      hipLaunchKernelGGL((bwd_uvw_kernel<LI, LS, LO, 2, NEED_P, POS, TAN, HESS, true>), grid, block, dyn, s, a);
    else
      hipLaunchKernelGGL((bwd_uvw_kernel<LI, LS, LO, 2, NEED_P, POS, TAN, HESS, false>), grid, block, dyn, s, a);
  } else {
    if (split)
      hipLaunchKernelGGL((bwd_uvw_kernel<LI, LS, LO, 4, NEED_P, POS, TAN, HESS, true>), grid, block, dyn, s, a);
    else
      hipLaunchKernelGGL((bwd_uvw_kernel<LI, LS, LO, 4, NEED_P, POS, TAN, HESS, false>), grid, block, dyn, s, a);
  }
  return hipGetLastError();
}

template <int LI, int LS, int LO, bool TAN, bool HESS>
hipError_t bwd_uvu_nb(const BwdUvuArgs& a, int nblocks, int ntiles, hipStream_t s) {
  dim3 grid(nblocks), block(64 * ntiles);
  const int rows = a.cp / 16;
  const size_t dyn = sizeof(float) * 64 * 3 * rows * ntiles;   // [ntiles][64][rows][3]
  if constexpr (!TAN && !HESS && kUvuFirst) {
    if (a.g.nb <= 8)
      hipLaunchKernelGGL((bwd_uvu_first_kernel<LI, LS, LO, 2>), grid, block, dyn, s, a);
    else
      hipLaunchKernelGGL((bwd_uvu_first_kernel<LI, LS, LO, 4>), grid, block, dyn, s, a);
  } else {
    if (a.g.nb <= 8)
      hipLaunchKernelGGL((bwd_uvu_kernel<LI, LS, LO, 2, TAN, HESS>), grid, block, dyn, s, a);
    else
      hipLaunchKernelGGL((bwd_uvu_kernel<LI, LS, LO, 4, TAN, HESS>), grid, block, dyn, s, a);
  }
  return hipGetLastError();
}

template <bool NEED_P, bool POS, bool TAN, bool HESS>
hipError_t launch_bwd_uvw_t(const BwdUvwArgs& a, int li, int lo, int nsend, int ntiles, hipStream_t s) {
#define ETPC_CALL(LI, LS, LO) bwd_uvw_nb<LI, LS, LO, NEED_P, POS, TAN, HESS>(a, nsend, ntiles, s)
  ETPC_TRIPLE_DISPATCH(li, a.ls, lo, ETPC_CALL)
#undef ETPC_CALL
}

template <bool TAN, bool HESS>
hipError_t launch_bwd_uvu_t(const BwdUvuArgs& a, int li, int lo, int nblocks, int ntiles, hipStream_t s) {
#define ETPC_CALL(LI, LS, LO) bwd_uvu_nb<LI, LS, LO, TAN, HESS>(a, nblocks, ntiles, s)
  ETPC_TRIPLE_DISPATCH(li, a.ls, lo, ETPC_CALL)
#undef ETPC_CALL
}

}  // namespace bwd_detail
}  // namespace etpc
