// Edge geometry device functions (fused into every traversal kernel; never stored).
//
// Edge vector r_e = p_sender - p_receiver (Sobek paper, Sec. 2, Eq. 8), minimum
// image in an orthorhombic box; distance r and direction u = r_e / r.
//
// Harmonics: real, component-normalized, evaluated from their homogeneous
// polynomial forms P_l at the unit vector (on the sphere P_l(u) = Y_l(u)).  The
// gradient with respect to the edge vector uses homogeneity of degree l:
//   dY_l/dr_e = (grad P_l(u) - l Y_l(u) u) / r.
// Radial bases: Gaussian  phi_b = exp(-(r - mu_b)^2 / (2 D^2));
//   Bessel  phi_b = sqrt(2/r_c) sin(b pi r / r_c) / r * f_p(r / r_c), b = 1..B,
//   f_p(t) = 1 - (p+1)(p+2)/2 t^p + p(p+2) t^(p+1) - p(p+1)/2 t^(p+2) (t < 1), else 0.
#pragma once

#include "common.hpp"

namespace etpc {

constexpr float kS3 = 1.7320508075688772f;
constexpr float kS5 = 2.23606797749979f;
constexpr float kS7 = 2.6457513110645907f;
constexpr float kS15 = 3.872983346207417f;
constexpr float kS42 = 6.48074069840786f;
constexpr float kS70 = 8.366600265340756f;
constexpr float kS105 = 10.246950765959598f;

__device__ inline void edge_vector(const GeomParams& g, const float* __restrict__ pos, int j, int i, float& rx,
                                   float& ry, float& rz) {
  rx = pos[3 * j + 0] - pos[3 * i + 0];
  ry = pos[3 * j + 1] - pos[3 * i + 1];
  rz = pos[3 * j + 2] - pos[3 * i + 2];
  if (g.periodic) {
    rx -= g.box[0] * rintf(rx * g.inv_box[0]);
    ry -= g.box[1] * rintf(ry * g.inv_box[1]);
    rz -= g.box[2] * rintf(rz * g.inv_box[2]);
  }
}

// Y_l(u) for one degree l (runtime), written into y[0..2l].
__device__ inline void sh_eval(int l, float x, float y, float z, float* __restrict__ out) {
  if (l == 0) {
    out[0] = 1.f;
  } else if (l == 1) {
    out[0] = kS3 * y;
    out[1] = kS3 * z;
    out[2] = kS3 * x;
  } else if (l == 2) {
    out[0] = kS15 * x * y;
    out[1] = kS15 * y * z;
    out[2] = 0.5f * kS5 * (2.f * z * z - x * x - y * y);
    out[3] = kS15 * x * z;
    out[4] = 0.5f * kS15 * (x * x - y * y);
  } else {
    const float x2 = x * x, y2 = y * y, z2 = z * z;
    out[0] = 0.25f * kS70 * y * (3.f * x2 - y2);
    out[1] = kS105 * x * y * z;
    out[2] = 0.25f * kS42 * y * (4.f * z2 - x2 - y2);
    out[3] = 0.5f * kS7 * z * (2.f * z2 - 3.f * x2 - 3.f * y2);
    out[4] = 0.25f * kS42 * x * (4.f * z2 - x2 - y2);
    out[5] = 0.5f * kS105 * z * (x2 - y2);
    out[6] = 0.25f * kS70 * x * (x2 - 3.f * y2);
  }
}

// Gradient of the homogeneous polynomial P_l at u: g[m][d], d = x,y,z.
__device__ inline void sh_poly_grad(int l, float x, float y, float z, float (*__restrict__ g)[3]) {
  if (l == 0) {
    g[0][0] = g[0][1] = g[0][2] = 0.f;
  } else if (l == 1) {
    g[0][0] = 0.f; g[0][1] = kS3; g[0][2] = 0.f;
    g[1][0] = 0.f; g[1][1] = 0.f; g[1][2] = kS3;
    g[2][0] = kS3; g[2][1] = 0.f; g[2][2] = 0.f;
  } else if (l == 2) {
    g[0][0] = kS15 * y; g[0][1] = kS15 * x; g[0][2] = 0.f;
    g[1][0] = 0.f; g[1][1] = kS15 * z; g[1][2] = kS15 * y;
    g[2][0] = -kS5 * x; g[2][1] = -kS5 * y; g[2][2] = 2.f * kS5 * z;
    g[3][0] = kS15 * z; g[3][1] = 0.f; g[3][2] = kS15 * x;
    g[4][0] = kS15 * x; g[4][1] = -kS15 * y; g[4][2] = 0.f;
  } else {
    const float x2 = x * x, y2 = y * y, z2 = z * z;
    const float a70 = 0.25f * kS70, a42 = 0.25f * kS42, a7 = 0.5f * kS7, a105 = 0.5f * kS105;
    g[0][0] = a70 * 6.f * x * y; g[0][1] = a70 * 3.f * (x2 - y2); g[0][2] = 0.f;
    g[1][0] = kS105 * y * z; g[1][1] = kS105 * x * z; g[1][2] = kS105 * x * y;
    g[2][0] = -a42 * 2.f * x * y; g[2][1] = a42 * (4.f * z2 - x2 - 3.f * y2); g[2][2] = a42 * 8.f * y * z;
    g[3][0] = -a7 * 6.f * x * z; g[3][1] = -a7 * 6.f * y * z; g[3][2] = a7 * (6.f * z2 - 3.f * x2 - 3.f * y2);
    g[4][0] = a42 * (4.f * z2 - 3.f * x2 - y2); g[4][1] = -a42 * 2.f * x * y; g[4][2] = a42 * 8.f * x * z;
    g[5][0] = a105 * 2.f * x * z; g[5][1] = -a105 * 2.f * y * z; g[5][2] = a105 * (x2 - y2);
    g[6][0] = a70 * 3.f * (x2 - y2); g[6][1] = -a70 * 6.f * x * y; g[6][2] = 0.f;
  }
}

// dY_l/dr_e[m][d] = (grad P_l(u) - l Y_l(u) u) / r
__device__ inline void sh_grad_r(int l, float x, float y, float z, float inv_r, const float* __restrict__ yv,
                                 float (*__restrict__ dy)[3]) {
  sh_poly_grad(l, x, y, z, dy);
  const int n = 2 * l + 1;
  for (int m = 0; m < n; ++m) {
    const float s = static_cast<float>(l) * yv[m];
    dy[m][0] = (dy[m][0] - s * x) * inv_r;
    dy[m][1] = (dy[m][1] - s * y) * inv_r;
    dy[m][2] = (dy[m][2] - s * z) * inv_r;
  }
}

// Hessian of the homogeneous polynomial P_l at u applied to v: h[m][d] = sum_e
// d^2 P_l / du_d du_e (u) v_e (differentiating the gradients above once more).
__device__ inline void sh_poly_hess_vec(int l, float x, float y, float z, float vx, float vy, float vz,
                                        float (*__restrict__ h)[3]) {
  if (l <= 1) {
    for (int m = 0; m < 2 * l + 1; ++m) h[m][0] = h[m][1] = h[m][2] = 0.f;
  } else if (l == 2) {
    h[0][0] = kS15 * vy; h[0][1] = kS15 * vx; h[0][2] = 0.f;
    h[1][0] = 0.f; h[1][1] = kS15 * vz; h[1][2] = kS15 * vy;
    h[2][0] = -kS5 * vx; h[2][1] = -kS5 * vy; h[2][2] = 2.f * kS5 * vz;
    h[3][0] = kS15 * vz; h[3][1] = 0.f; h[3][2] = kS15 * vx;
    h[4][0] = kS15 * vx; h[4][1] = -kS15 * vy; h[4][2] = 0.f;
  } else {
    const float a70 = 0.25f * kS70, a42 = 0.25f * kS42, a7 = 0.5f * kS7, a105 = 0.5f * kS105;
    const float xy = y * vx + x * vy, yz = z * vy + y * vz, xz = z * vx + x * vz;
    h[0][0] = a70 * 6.f * xy; h[0][1] = a70 * 6.f * (x * vx - y * vy); h[0][2] = 0.f;
    h[1][0] = kS105 * yz; h[1][1] = kS105 * xz; h[1][2] = kS105 * xy;
    h[2][0] = -a42 * 2.f * xy; h[2][1] = a42 * (8.f * z * vz - 2.f * x * vx - 6.f * y * vy); h[2][2] = a42 * 8.f * yz;
    h[3][0] = -a7 * 6.f * xz; h[3][1] = -a7 * 6.f * yz; h[3][2] = a7 * (12.f * z * vz - 6.f * x * vx - 6.f * y * vy);
    h[4][0] = a42 * (8.f * z * vz - 6.f * x * vx - 2.f * y * vy); h[4][1] = -a42 * 2.f * xy; h[4][2] = a42 * 8.f * xz;
    h[5][0] = a105 * 2.f * xz; h[5][1] = -a105 * 2.f * yz; h[5][2] = a105 * 2.f * (x * vx - y * vy);
    h[6][0] = a70 * 6.f * (x * vx - y * vy); h[6][1] = -a70 * 6.f * xy; h[6][2] = 0.f;
  }
}

// Directional derivative of dY_l/dr_e (above) along the edge-vector tangent rdot:
//   with rho_dot = u . rdot and u_dot = (rdot - u rho_dot) / r,
//   d(dY/dr) = (H_P(u) u_dot - l (grad P(u) . u_dot) u - l Y u_dot) / r - dY rho_dot / r.
__device__ inline void sh_grad_r_dir(int l, float x, float y, float z, float inv_r, const float* __restrict__ yv,
                                     const float (*__restrict__ dy)[3], float udx, float udy, float udz,
                                     float rho_dot, float (*__restrict__ ddy)[3]) {
  float gp[7][3], hv[7][3];
  sh_poly_grad(l, x, y, z, gp);
  sh_poly_hess_vec(l, x, y, z, udx, udy, udz, hv);
  const float fl = static_cast<float>(l);
  for (int m = 0; m < 2 * l + 1; ++m) {
    const float gu = gp[m][0] * udx + gp[m][1] * udy + gp[m][2] * udz;
    ddy[m][0] = (hv[m][0] - fl * gu * x - fl * yv[m] * udx) * inv_r - dy[m][0] * rho_dot * inv_r;
    ddy[m][1] = (hv[m][1] - fl * gu * y - fl * yv[m] * udy) * inv_r - dy[m][1] * rho_dot * inv_r;
    ddy[m][2] = (hv[m][2] - fl * gu * z - fl * yv[m] * udz) * inv_r - dy[m][2] * rho_dot * inv_r;
  }
}

// phi[0..NB) (zero-padded beyond nb); if dphi != nullptr also d phi / d r.
// If ddphi != nullptr also d^2 phi / d r^2 (Gaussian: (4 a^2 t^2 - 2 a) phi with
// a = 1 / (2 D^2); Bessel: product rule on the bare sin(k r) / r and the envelope).
template <int NB>
__device__ inline void radial_eval(const GeomParams& g, float r, float* __restrict__ phi, float* __restrict__ dphi,
                                   float* __restrict__ ddphi = nullptr) {
  if (g.radial == ETPC_RADIAL_GAUSSIAN) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < g.nb) {
        const float t = r - (g.r_lo + b * g.gauss_d);
        const float e = __expf(-t * t * g.gauss_inv2d2);
        phi[b] = e;
        if (dphi) dphi[b] = -2.f * g.gauss_inv2d2 * t * e;
        if (ddphi) ddphi[b] = (4.f * g.gauss_inv2d2 * g.gauss_inv2d2 * t * t - 2.f * g.gauss_inv2d2) * e;
      } else {
        phi[b] = 0.f;
        if (dphi) dphi[b] = 0.f;
        if (ddphi) ddphi[b] = 0.f;
      }
    }
  } else {
    const float rc = g.r_hi;
    const float t = r / rc;
    float f = 0.f, fp = 0.f, fpp = 0.f;
    if (t < 1.f) {
      const int p = g.poly_p;
      const float pf = static_cast<float>(p);
      const float tp2 = __powf(t, pf - 2.f);  // t^(p-2), t > 0
      const float tp1 = tp2 * t;
      const float tp = tp1 * t;
      const float a = 0.5f * (pf + 1.f) * (pf + 2.f), bb = pf * (pf + 2.f), c = 0.5f * pf * (pf + 1.f);
      f = 1.f - a * tp + bb * tp * t - c * tp * t * t;
      fp = (-a * pf * tp1 + bb * (pf + 1.f) * tp - c * (pf + 2.f) * tp * t) / rc;
      fpp = (-a * pf * (pf - 1.f) * tp2 + bb * (pf + 1.f) * pf * tp1 - c * (pf + 2.f) * (pf + 1.f) * tp) /
            (rc * rc);
    }
    const float amp = sqrtf(2.f / rc);
    const float inv_r = 1.f / r;
    const float w = 3.14159265358979323846f / rc;
    // sin(b w r), cos(b w r) for b = 1..B by the Chebyshev recurrence
    // s_(b+1) = 2 cos(w r) s_b - s_(b-1), and the same for the cosines
    float s1, c1;
    sincosf(w * r, &s1, &c1);
    float sp = 0.f, sc = s1, cpv = 1.f, cc = c1;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < g.nb) {
        const float k = w * (b + 1);
        const float bare = amp * sc * inv_r;
        phi[b] = bare * f;
        if (dphi) {
          const float dbare = amp * (k * cc - sc * inv_r) * inv_r;
          dphi[b] = dbare * f + bare * fp;
          if (ddphi) {
            const float ddbare = amp * (-k * k * sc - 2.f * k * cc * inv_r + 2.f * sc * inv_r * inv_r) * inv_r;
            ddphi[b] = ddbare * f + 2.f * dbare * fp + bare * fpp;
          }
        }
      } else {
        phi[b] = 0.f;
        if (dphi) dphi[b] = 0.f;
        if (ddphi) ddphi[b] = 0.f;
      }
      const float sn = 2.f * c1 * sc - sp;
      const float cn = 2.f * c1 * cc - cpv;
      sp = sc;
      sc = sn;
      cpv = cc;
      cc = cn;
    }
  }
}

}  // namespace etpc
