// Dense fp32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2f32).
//
// Used for the channel-space products of the Sobek paper (Sec. 4, Eq. 34-36):
// m = S W (forward), and the node-side products of the sender-factorized
// backward: Xt = x W, x_bar = P W^T, W_bar = x^T P.  Rows of A and C are given
// through a RowMap so ir_mul feature blocks ((node, m) rows) are read and written
// in place.  A 64x64 output tile per 256-thread workgroup, four wavefronts of
// 32x32, K staged through LDS in slices of 16 (double-buffered through registers).
#include "kernels.hpp"

namespace etpc {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BM = 64, BN = 64, BK = 16;

__device__ inline int64_t rowoff(const RowMap& m, int r) {
  const int q = r / m.div;
  return static_cast<int64_t>(q) * m.s1 + static_cast<int64_t>(r - q * m.div) * m.s2;
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmArgs a) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid & 1, wn = wid >> 1;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int kz0 = blockIdx.z * a.k_split;
  const int kz1 = min(a.K, kz0 + a.k_split);
  float* C = a.C + static_cast<int64_t>(blockIdx.z) * a.c_split_stride;

  // load assignments
  const int a_row = tid >> 2, a_k4 = (tid & 3) * 4;      // K-contiguous A: row, 4 k's
  const int t_k = tid >> 4, t_c4 = (tid & 15) * 4;       // k-major: k, 4 columns
  int64_t a_rowoff = 0;
  const bool a_row_ok = (m0 + a_row) < a.M;
  if (!a.a_mcontig && a_row_ok) a_rowoff = rowoff(a.amap, m0 + a_row);

  float ra[4], rb[4];
  auto load = [&](int k0) {
    if (!a.a_mcontig) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = k0 + a_k4 + t;
        ra[t] = (a_row_ok && k < kz1) ? a.A[a_rowoff + k] : 0.f;
      }
    } else {
      const int k = k0 + t_k;
      const bool kok = k < kz1;
      const int64_t ko = kok ? rowoff(a.amap, k) : 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + t_c4 + t;
        ra[t] = (kok && m < a.M) ? a.A[ko + m] : 0.f;
      }
    }
    const int k = k0 + t_k;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = n0 + t_c4 + t;
      rb[t] = (k < kz1 && n < a.N) ? a.B[static_cast<int64_t>(k) * a.ldb + n] : 0.f;
    }
  };
  auto store = [&]() {
    if (!a.a_mcontig) {
#pragma unroll
      for (int t = 0; t < 4; ++t) As[a_k4 + t][a_row] = ra[t];
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) As[t_k][t_c4 + t] = ra[t];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) Bs[t_k][t_c4 + t] = rb[t];
  };

  f16v acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (kz0 < kz1) load(kz0);
  for (int k0 = kz0; k0 < kz1; k0 += BK) {
    store();
    __syncthreads();
    if (k0 + BK < kz1) load(k0 + BK);
    const int am = wm * 32 + (lane & 31), bn = wn * 32 + (lane & 31), kh = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[kk + kh][am], Bs[kk + kh][bn], acc, 0, 0, 0);
    }
    __syncthreads();
  }
  const int n = n0 + wn * 32 + (lane & 31);
  if (n < a.N) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m < a.M) {
        float* p = C + rowoff(a.cmap, m) + n;
        *p = a.beta ? (*p + acc[r]) : acc[r];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int splits, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  dim3 grid((a.M + BM - 1) / BM, (a.N + BN - 1) / BN, splits), block(256);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace etpc
