// Planner (host): validation, path enumeration, real coupling tensors, offsets.
//
// Path enumeration follows the Clebsch-Gordan selection rule of the Sobek paper
// (Sec. 2, Eq. 5): |l_in - l_sh| <= l_out <= l_in + l_sh, parity_out =
// parity_in * (-1)^l_sh.  Weight widths follow Eq. 9-10 (uvw: C_in C_out per
// basis, uvu: C_in per basis, Eq. 7).
//
// Coupling tensors: the complex Clebsch-Gordan coefficients come from Racah's
// closed formula; they are moved to the real harmonic basis of this library
// with the unitary change of basis U (rows: real m, columns: complex mu,
// Condon-Shortley phase), c = U3 . C . conj(U1) conj(U2), which is exactly real
// or exactly imaginary; the nonzero part is scaled so each output column has
// unit norm and signed so the first nonzero entry (C order) is positive.
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <complex>
#include <cstring>
#include <set>
#include <string>
#include <tuple>

namespace etpc {

namespace {

thread_local std::string g_error;

double fact(int n) {
  double r = 1.0;
  for (int i = 2; i <= n; ++i) r *= i;
  return r;
}

// <j1 m1 j2 m2 | J M>, Racah's formula (integer angular momenta).
double cg_complex(int j1, int m1, int j2, int m2, int J, int M) {
  if (m1 + m2 != M) return 0.0;
  if (std::abs(m1) > j1 || std::abs(m2) > j2 || std::abs(M) > J) return 0.0;
  if (J < std::abs(j1 - j2) || J > j1 + j2) return 0.0;
  const double pre = std::sqrt((2.0 * J + 1.0) * fact(J + j1 - j2) * fact(J - j1 + j2) * fact(j1 + j2 - J) /
                               fact(j1 + j2 + J + 1));
  const double pre2 = std::sqrt(fact(J + M) * fact(J - M) * fact(j1 - m1) * fact(j1 + m1) * fact(j2 - m2) *
                                fact(j2 + m2));
  double sum = 0.0;
  for (int k = 0; k <= j1 + j2 + J; ++k) {
    const int a = j1 + j2 - J - k, b = j1 - m1 - k, c = j2 + m2 - k, d = J - j2 + m1 + k, e = J - j1 - m2 + k;
    if (a < 0 || b < 0 || c < 0 || d < 0 || e < 0) continue;
    const double term = 1.0 / (fact(k) * fact(a) * fact(b) * fact(c) * fact(d) * fact(e));
    sum += (k % 2 == 0) ? term : -term;
  }
  return pre * pre2 * sum;
}

// U[m][mu] for degree l: real harmonic index m = -l..l in terms of complex ones.
void real_from_complex(int l, std::complex<double>* U) {
  const int n = 2 * l + 1;
  for (int i = 0; i < n * n; ++i) U[i] = 0.0;
  const double s = 1.0 / std::sqrt(2.0);
  for (int m = -l; m <= l; ++m) {
    const int r = m + l;
    if (m == 0) {
      U[r * n + l] = 1.0;
    } else if (m > 0) {
      const double sg = (m % 2 == 0) ? 1.0 : -1.0;
      U[r * n + (m + l)] = sg * s;
      U[r * n + (-m + l)] = s;
    } else {
      const int k = -m;
      const double sg = (k % 2 == 0) ? 1.0 : -1.0;
      U[r * n + (-k + l)] = std::complex<double>(0.0, s);
      U[r * n + (k + l)] = std::complex<double>(0.0, -sg * s);
    }
  }
}

}  // namespace

void set_error(const std::string& msg) { g_error = msg; }
const char* last_error() { return g_error.c_str(); }

bool real_cg_racah(int l1, int l2, int l3, double* out) {
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
  std::fill(out, out + n1 * n2 * n3, 0.0);
  if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) return false;
  std::complex<double> U1[49], U2[49], U3[49];
  real_from_complex(l1, U1);
  real_from_complex(l2, U2);
  real_from_complex(l3, U3);
  std::vector<std::complex<double>> c(n1 * n2 * n3, 0.0);
  for (int a = 0; a < n1; ++a)
    for (int b = 0; b < n2; ++b)
      for (int m = 0; m < n3; ++m) {
        std::complex<double> acc = 0.0;
        for (int mu1 = -l1; mu1 <= l1; ++mu1)
          for (int mu2 = -l2; mu2 <= l2; ++mu2) {
            const int mu3 = mu1 + mu2;
            if (std::abs(mu3) > l3) continue;
            const double cc = cg_complex(l1, mu1, l2, mu2, l3, mu3);
            if (cc == 0.0) continue;
            acc += U3[m * n3 + (mu3 + l3)] * cc * std::conj(U1[a * n1 + (mu1 + l1)]) *
                   std::conj(U2[b * n2 + (mu2 + l2)]);
          }
        c[(a * n2 + b) * n3 + m] = acc;
      }
  double re = 0.0, im = 0.0;
  for (auto& v : c) {
    re = std::max(re, std::abs(v.real()));
    im = std::max(im, std::abs(v.imag()));
  }
  const bool use_re = re >= im;
  double norm2 = 0.0;
  for (size_t i = 0; i < c.size(); ++i) {
    out[i] = use_re ? c[i].real() : c[i].imag();
    norm2 += out[i] * out[i];
  }
  const double scale = std::sqrt(static_cast<double>(n3) / norm2);
  double sign = 1.0;
  for (size_t i = 0; i < c.size(); ++i) {
    if (std::abs(out[i] * scale) > 1e-9) {
      sign = out[i] < 0 ? -1.0 : 1.0;
      break;
    }
  }
  for (size_t i = 0; i < c.size(); ++i) {
    out[i] *= scale * sign;
    if (std::abs(out[i]) < 1e-14) out[i] = 0.0;
  }
  return true;
}

}  // namespace etpc

etpc::GeomParams etpc_plan_s::geom() const {
  etpc::GeomParams g{};
  g.radial = radial;
  g.nb = n_basis;
  g.r_lo = r_lo;
  g.r_hi = r_hi;
  if (radial == ETPC_RADIAL_GAUSSIAN) {
    const double d = (static_cast<double>(r_hi) - r_lo) / (n_basis - 1);
    g.gauss_d = static_cast<float>(d);
    g.gauss_inv2d2 = static_cast<float>(1.0 / (2.0 * d * d));
  }
  g.poly_p = poly_p;
  g.periodic = periodic ? 1 : 0;
  for (int d = 0; d < 3; ++d) {
    g.box[d] = box[d];
    g.inv_box[d] = periodic ? static_cast<float>(1.0 / box[d]) : 0.f;
  }
  return g;
}

namespace {

bool selection_ok(int li, int pi, int ls, int lo, int po) {
  const int psh = (ls % 2 == 0) ? 1 : -1;
  return std::abs(li - ls) <= lo && lo <= li + ls && po == pi * psh;
}

etpc_status check_irreps(const etpc_irrep* v, int n, bool mul_needed, const char* what) {
  if (n < 1 || v == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, std::string(what) + ": empty or null irreps");
  for (int i = 0; i < n; ++i) {
    if (mul_needed && v[i].mul < 1)
      ETPC_FAIL(ETPC_ERR_INVALID_ARG, std::string(what) + ": multiplicity must be >= 1");
    if (v[i].l < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, std::string(what) + ": negative l");
    if (v[i].l > etpc::kMaxL) ETPC_FAIL(ETPC_ERR_UNSUPPORTED, std::string(what) + ": l > 3 is not supported");
    if (v[i].parity != 1 && v[i].parity != -1)
      ETPC_FAIL(ETPC_ERR_INVALID_ARG, std::string(what) + ": parity must be +1 or -1");
  }
  return ETPC_OK;
}

}  // namespace

extern "C" {

const char* etpc_last_error(void) { return etpc::last_error(); }

etpc_status etpc_plan_create(const etpc_spec* s, etpc_plan* out) {
  using etpc::PathInfo;
  if (s == nullptr || out == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null spec or output handle");
  *out = nullptr;
  if (s->mode != ETPC_UVW && s->mode != ETPC_UVU) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "mode must be UVW or UVU");
  if (s->out_per_path && s->mode != ETPC_UVU)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "out_per_path is only defined for uvu");
  etpc_status st = check_irreps(s->in, s->n_in, true, "input");
  if (st != ETPC_OK) return st;
  st = check_irreps(s->out, s->n_out, !s->out_per_path, "output");
  if (st != ETPC_OK) return st;
  if (s->lmax_sh < 0) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "lmax_sh must be >= 0");
  if (s->lmax_sh > etpc::kMaxL) ETPC_FAIL(ETPC_ERR_UNSUPPORTED, "lmax_sh > 3 is not supported");
  if (s->radial != ETPC_RADIAL_GAUSSIAN && s->radial != ETPC_RADIAL_BESSEL_POLY)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "unknown radial basis");
  if (s->n_basis < 1) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "n_basis must be >= 1");
  if (s->n_basis > etpc::kMaxBasis) ETPC_FAIL(ETPC_ERR_UNSUPPORTED, "n_basis > 16 is not supported");
  if (s->radial == ETPC_RADIAL_GAUSSIAN) {
    if (s->n_basis < 2) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "a Gaussian basis needs n_basis >= 2");
    if (!(s->r_hi > s->r_lo)) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "Gaussian basis needs r_hi > r_lo");
  } else {
    if (!(s->r_hi > 0.f)) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "Bessel basis needs a positive cutoff r_hi");
    if (s->poly_p < 1) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "poly_p must be >= 1");
  }
  const bool any_box = s->box[0] != 0.f || s->box[1] != 0.f || s->box[2] != 0.f;
  if (any_box && !(s->box[0] > 0.f && s->box[1] > 0.f && s->box[2] > 0.f))
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "box must be all zero (open) or all positive");
  if (s->gemm_precision != ETPC_GEMM_FP32 && s->gemm_precision != ETPC_GEMM_BF16 &&
      s->gemm_precision != ETPC_GEMM_FP16)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "unknown gemm_precision");
  if (s->lanes < 0 || s->lanes > etpc::kLanes)
    ETPC_FAIL(ETPC_ERR_INVALID_ARG, "lanes must be 0 (default) or 1.." + std::to_string(etpc::kLanes));

  auto p = new etpc_plan_s();
  p->in.assign(s->in, s->in + s->n_in);
  p->lmax_sh = s->lmax_sh;
  p->mode = s->mode;
  p->radial = s->radial;
  p->n_basis = s->n_basis;
  p->poly_p = s->poly_p;
  p->r_lo = s->r_lo;
  p->r_hi = s->r_hi;
  p->periodic = any_box;
  for (int d = 0; d < 3; ++d) p->box[d] = s->box[d];
  p->gemm_precision = s->gemm_precision;
  p->lanes = s->lanes == 0 ? etpc::kLanes : s->lanes;

  std::vector<std::tuple<int, int, int>> instr;
  if (s->out_per_path) {
    if (s->n_instr != 0) {
      delete p;
      ETPC_FAIL(ETPC_ERR_INVALID_ARG, "out_per_path builds its own instruction list");
    }
    for (int k = 0; k < s->n_in; ++k)
      for (int ls = 0; ls <= s->lmax_sh; ++ls)
        for (int a = 0; a < s->n_out; ++a)
          if (selection_ok(s->in[k].l, s->in[k].parity, ls, s->out[a].l, s->out[a].parity)) {
            instr.emplace_back(k, ls, static_cast<int>(p->out.size()));
            p->out.push_back(etpc_irrep{s->in[k].mul, s->out[a].l, s->out[a].parity});
          }
  } else {
    p->out.assign(s->out, s->out + s->n_out);
    if (s->n_instr > 0) {
      if (s->instr == nullptr) {
        delete p;
        ETPC_FAIL(ETPC_ERR_INVALID_ARG, "n_instr > 0 but instr is null");
      }
      std::set<std::tuple<int, int, int>> seen;
      for (int t = 0; t < s->n_instr; ++t) {
        const etpc_instr& it = s->instr[t];
        if (it.in_block < 0 || it.in_block >= s->n_in || it.out_block < 0 || it.out_block >= s->n_out ||
            it.l_sh < 0 || it.l_sh > s->lmax_sh) {
          delete p;
          ETPC_FAIL(ETPC_ERR_INVALID_ARG, "instruction index out of range");
        }
        auto key = std::make_tuple(it.in_block, it.l_sh, it.out_block);
        if (!seen.insert(key).second) {
          delete p;
          ETPC_FAIL(ETPC_ERR_INVALID_ARG, "duplicate instruction");
        }
        instr.push_back(key);
      }
    } else if (s->n_instr < 0) {
      delete p;
      ETPC_FAIL(ETPC_ERR_INVALID_ARG, "n_instr must be >= 0");
    } else {
      for (int g = 0; g < s->n_out; ++g)
        for (int k = 0; k < s->n_in; ++k)
          for (int ls = 0; ls <= s->lmax_sh; ++ls)
            if (selection_ok(s->in[k].l, s->in[k].parity, ls, s->out[g].l, s->out[g].parity))
              instr.emplace_back(k, ls, g);
    }
  }
  for (auto& t : instr) {
    const auto& a = p->in[std::get<0>(t)];
    const auto& b = p->out[std::get<2>(t)];
    if (!selection_ok(a.l, a.parity, std::get<1>(t), b.l, b.parity)) {
      delete p;
      ETPC_FAIL(ETPC_ERR_INVALID_PATH, "instruction violates the Clebsch-Gordan selection rule");
    }
    if (p->mode == ETPC_UVU && a.mul != b.mul) {
      delete p;
      ETPC_FAIL(ETPC_ERR_INVALID_PATH, "uvu instruction needs equal input and output multiplicity");
    }
  }
  if (static_cast<int>(instr.size()) > etpc::kMaxPaths) {
    delete p;
    ETPC_FAIL(ETPC_ERR_UNSUPPORTED, "more than 64 paths");
  }
  // plan order: (out_block, in_block, l_sh)
  std::sort(instr.begin(), instr.end(), [](const auto& x, const auto& y) {
    return std::make_tuple(std::get<2>(x), std::get<0>(x), std::get<1>(x)) <
           std::make_tuple(std::get<2>(y), std::get<0>(y), std::get<1>(y));
  });
  int64_t o = 0;
  for (auto& b : p->in) {
    p->xoff.push_back(o);
    o += static_cast<int64_t>(b.mul) * (2 * b.l + 1);
  }
  p->x_dim = o;
  o = 0;
  for (auto& b : p->out) {
    p->zoff.push_back(o);
    o += static_cast<int64_t>(b.mul) * (2 * b.l + 1);
  }
  p->z_dim = o;
  p->by_out.assign(p->out.size(), {});
  p->by_in.assign(p->in.size(), {});
  int64_t woff = 0;
  for (auto& t : instr) {
    PathInfo pi{};
    pi.in_block = std::get<0>(t);
    pi.l_sh = std::get<1>(t);
    pi.out_block = std::get<2>(t);
    pi.l_in = p->in[pi.in_block].l;
    pi.l_out = p->out[pi.out_block].l;
    pi.c_in = p->in[pi.in_block].mul;
    pi.c_out = p->out[pi.out_block].mul;
    pi.w_off = woff;
    pi.w_numel = static_cast<int64_t>(p->n_basis) * pi.c_in * (p->mode == ETPC_UVW ? pi.c_out : 1);
    woff += pi.w_numel;
    etpc::real_cg_racah(pi.l_in, pi.l_sh, pi.l_out, pi.cg);
    const int ni = 2 * pi.l_in + 1, ns = 2 * pi.l_sh + 1, no = 2 * pi.l_out + 1;
    std::memset(&pi.cgf, 0, sizeof(pi.cgf));
    for (int a = 0; a < ni; ++a)
      for (int b = 0; b < ns; ++b)
        for (int m = 0; m < no; ++m) pi.cgf.c[(a * 7 + b) * no + m] = static_cast<float>(pi.cg[(a * ns + b) * no + m]);
    const int idx = static_cast<int>(p->paths.size());
    pi.pos_in_group = static_cast<int>(p->by_out[pi.out_block].size());
    pi.pos_in_block = static_cast<int>(p->by_in[pi.in_block].size());
    p->by_out[pi.out_block].push_back(idx);
    p->by_in[pi.in_block].push_back(idx);
    p->paths.push_back(pi);
  }
  p->w_numel = woff;
  for (auto& pi : p->paths) {
    if (p->mode == ETPC_UVW) {
      int64_t s = 0;
      for (int q : p->by_out[pi.out_block]) s += p->paths[q].c_in;
      pi.fan_in = static_cast<int32_t>(s * p->n_basis);
    } else {
      pi.fan_in = p->n_basis;
    }
  }
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (p->x_dim > lim || p->z_dim > lim || p->w_numel > lim) {
    delete p;
    ETPC_FAIL(ETPC_ERR_OVERFLOW, "feature or weight width exceeds int32");
  }
  *out = p;
  return ETPC_OK;
}

void etpc_plan_destroy(etpc_plan plan) { delete plan; }

etpc_status etpc_plan_info(etpc_plan p, int64_t* x_dim, int64_t* z_dim, int64_t* w_numel, int32_t* n_paths) {
  if (p == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null plan");
  if (x_dim) *x_dim = p->x_dim;
  if (z_dim) *z_dim = p->z_dim;
  if (w_numel) *w_numel = p->w_numel;
  if (n_paths) *n_paths = static_cast<int32_t>(p->paths.size());
  return ETPC_OK;
}

etpc_status etpc_plan_path(etpc_plan p, int32_t i, int32_t* in_block, int32_t* l_sh, int32_t* out_block,
                           int32_t* l_in, int32_t* l_out, int64_t* x_off, int64_t* z_off, int64_t* w_off,
                           int64_t* w_numel, int32_t* fan_in) {
  if (p == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null plan");
  if (i < 0 || i >= static_cast<int32_t>(p->paths.size())) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "path index out of range");
  const auto& q = p->paths[i];
  if (in_block) *in_block = q.in_block;
  if (l_sh) *l_sh = q.l_sh;
  if (out_block) *out_block = q.out_block;
  if (l_in) *l_in = q.l_in;
  if (l_out) *l_out = q.l_out;
  if (x_off) *x_off = p->xoff[q.in_block];
  if (z_off) *z_off = p->zoff[q.out_block];
  if (w_off) *w_off = q.w_off;
  if (w_numel) *w_numel = q.w_numel;
  if (fan_in) *fan_in = q.fan_in;
  return ETPC_OK;
}

etpc_status etpc_plan_out_irrep(etpc_plan p, int32_t b, int32_t* n_out, etpc_irrep* irrep) {
  if (p == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null plan");
  if (n_out) *n_out = static_cast<int32_t>(p->out.size());
  if (irrep) {
    if (b < 0 || b >= static_cast<int32_t>(p->out.size())) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "block index out of range");
    *irrep = p->out[b];
  }
  return ETPC_OK;
}

etpc_status etpc_plan_cg(etpc_plan p, int32_t i, double* out) {
  if (p == nullptr || out == nullptr) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "null plan or output");
  if (i < 0 || i >= static_cast<int32_t>(p->paths.size())) ETPC_FAIL(ETPC_ERR_INVALID_ARG, "path index out of range");
  const auto& q = p->paths[i];
  const int n = (2 * q.l_in + 1) * (2 * q.l_sh + 1) * (2 * q.l_out + 1);
  std::memcpy(out, q.cg, sizeof(double) * n);
  return ETPC_OK;
}

}  // extern "C"
