// Dense GEMM on the gfx950 matrix cores: fp32 (v_mfma_f32_32x32x2f32), or with bf16 or
// fp16 operands and fp32 accumulation (v_mfma_f32_32x32x16_bf16 / _f16) when the plan asks.
//
// Used for the channel-space products of the Sobek paper (Sec. 4, Eq. 34-36):
// m = S W (forward), and the node-side products of the sender-factorized
// backward: Xt = x W, x_bar = P W^T, W_bar = x^T P.  Rows of A and C are given
// through a RowMap so ir_mul feature blocks ((node, m) rows) are read and written
// in place.  Four 32x32 wavefront blocks per 256-thread workgroup (64x64, or 128x32 /
// 32x128 against a 32-channel side), K staged through LDS in slices of 32 with the
// next slice's global loads in flight during the current slice's MFMAs.  Long-K
// products split K across workgroups; the partial tiles are summed in a fixed order by
// a second kernel.
#include "kernels.hpp"

namespace etpc {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BK = 32;

__device__ inline int64_t rowoff(const RowMap& m, int r) {
  const int q = static_cast<int>((__umulhi(static_cast<uint32_t>(r), m.magic) + static_cast<uint32_t>(r)) >> m.shift);
  return static_cast<int64_t>(q) * m.s1 + static_cast<int64_t>(r - q * m.div) * m.s2;
}

// One workgroup of four wavefronts arranged WGM x WGN computes a (32 WGM) x (32 WGN) tile
// of C: 64 x 64, or 128 x 32 / 32 x 128 against a 32-channel side.  Per K slice of KB
// values every thread moves groups of 4 consecutive elements (float4 when aligned) from
// global memory into LDS tiles As[k][m] and Bs[k][n]; the 32x32x2 MFMA reads k = kk + kh
// from lane half kh (32 consecutive m or n of one row: no bank conflict).  Groups along m
// or n (B, and an m-contiguous A) go in as one 16-byte LDS store (row stride 32 WGM + 4 or
// 32 WGN + 4).  A K-contiguous A is read with eight consecutive lanes per row (full
// 128-byte row segments) and stored transposed, four 4-byte stores per group, into rows
// of odd stride 32 WGM + 1, so the 32 lanes of a half-wave (eight k groups x four rows)
// hit 32 distinct banks.  MC: A is m-contiguous (GemmArgs::a_mcontig).  The wave budget
// keeps the 64 x 64 tile within 64 VGPRs (eight waves per SIMD: the short-K node GEMMs
// are latency-bound) and the narrow tiles within 80.
template <int WGM, int WGN, bool MC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WGM == 2 ? 8 : 6))) void gemm_f32_kernel(
    const GemmArgs a) {
  constexpr int BM = 32 * WGM, BN = 32 * WGN, KB = kGemmBK;
  static_assert(KB == 32 || KB == 64, "K slice of 32 or 64");
  static_assert(WGM * WGN == 4, "four wavefronts per workgroup");
  constexpr int AG = BM * KB / 1024, BG = BN * KB / 1024;  // float4 groups per thread and slice
  constexpr int LKM = MC ? BM + 4 : BM + 1, LKN = BN + 4;   // As[k][m] / Bs[k][n] row strides
  // the operand tiles, then (after the last slice) the C tile on its way out (row stride
  // BN + 4: the MFMA-layout writes and the 16-byte row reads are both free of bank conflicts)
  constexpr int LC = BN + 4;
  constexpr int kSmem = KB * LKM + KB * LKN > BM * LC ? KB * LKM + KB * LKN : BM * LC;
  __shared__ __attribute__((aligned(16))) float smem[kSmem];
  float* const As = smem;
  float* const Bs = smem + KB * LKM;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid % WGM, wn = wid / WGM;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int kz0 = blockIdx.z * a.k_split;
  const int kz1 = min(a.K, kz0 + a.k_split);
  float* C = a.C + static_cast<int64_t>(blockIdx.z) * a.c_split_stride;
  const bool vec = a.vec4 != 0;

  // group h of this thread (g = tid + 256 h): K-contiguous A -> row g / (KB / 4),
  // k4 = 4 (g % (KB / 4)); m-contiguous A -> k = g / (BM / 4), m4 = 4 (g % (BM / 4));
  // B -> k = g / (BN / 4), n4 = 4 (g % (BN / 4)).  Only the A row offsets are kept.
  int64_t a_off[AG];
  bool a_ok[AG];
#pragma unroll
  for (int h = 0; h < AG; ++h) {
    a_off[h] = 0;
    a_ok[h] = false;
    if constexpr (!MC) {
      const int m = m0 + (tid + 256 * h) / (KB / 4);
      a_ok[h] = m < a.M;
      if (a_ok[h]) a_off[h] = rowoff(a.amap, m);
    }
  }
  float4 ra[AG], rb[BG];
  auto load4 = [&](const float* p, int valid) -> float4 {
    if (valid == 4 && vec) return *reinterpret_cast<const float4*>(p);
    float4 v;
    v.x = valid > 0 ? p[0] : 0.f;
    v.y = valid > 1 ? p[1] : 0.f;
    v.z = valid > 2 ? p[2] : 0.f;
    v.w = valid > 3 ? p[3] : 0.f;
    return v;
  };
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < AG; ++h) {
      const int g = tid + 256 * h;
      if constexpr (!MC) {
        const int k = k0 + (g % (KB / 4)) * 4;
        ra[h] = load4(a.A + a_off[h] + k, a_ok[h] ? min(4, kz1 - k) : 0);
      } else {
        const int k = k0 + g / (BM / 4);
        const int m = m0 + (g % (BM / 4)) * 4;
        const int valid = k < kz1 ? min(4, a.M - m) : 0;
        ra[h] = load4(a.A + (valid > 0 ? rowoff(a.amap, k) : 0) + m, valid);
      }
    }
#pragma unroll
    for (int h = 0; h < BG; ++h) {
      const int g = tid + 256 * h;
      const int k = k0 + g / (BN / 4);
      const int n = n0 + (g % (BN / 4)) * 4;
      const int valid = k < kz1 ? min(4, a.N - n) : 0;
      rb[h] = load4(a.B + static_cast<int64_t>(k < kz1 ? k : 0) * a.ldb + n, valid);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int h = 0; h < AG; ++h) {
      const int g = tid + 256 * h;
      if constexpr (!MC) {
        const int row = g / (KB / 4), k4 = (g % (KB / 4)) * 4;
        As[k4 * LKM + row] = ra[h].x;
        As[(k4 + 1) * LKM + row] = ra[h].y;
        As[(k4 + 2) * LKM + row] = ra[h].z;
        As[(k4 + 3) * LKM + row] = ra[h].w;
      } else {
        *reinterpret_cast<float4*>(As + (g / (BM / 4)) * LKM + (g % (BM / 4)) * 4) = ra[h];
      }
    }
#pragma unroll
    for (int h = 0; h < BG; ++h) {
      const int g = tid + 256 * h;
      *reinterpret_cast<float4*>(Bs + (g / (BN / 4)) * LKN + (g % (BN / 4)) * 4) = rb[h];
    }
  };

  f16v acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (kz0 < kz1) load(kz0);
  const int am = wm * 32 + (lane & 31), bn = wn * 32 + (lane & 31), kh = lane >> 5;
  const int a_rd = kh * LKM + am, b_rd = kh * LKN + bn;   // row kh of As[k][m] / Bs[k][n]
  for (int k0 = kz0; k0 < kz1; k0 += KB) {
    store();
    __syncthreads();
    if (k0 + KB < kz1) load(k0 + KB);
#pragma unroll
    for (int kk = 0; kk < KB; kk += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[a_rd + kk * LKM], Bs[b_rd + kk * LKN], acc, 0, 0, 0);
    __syncthreads();
  }
  // C leaves through LDS (the last slice ended with a barrier, so the operand tiles are
  // free): each thread writes four consecutive columns of a row as one 16-byte store, where
  // the MFMA layout would give 4-byte stores of 32-column half rows (16 store instructions
  // per wave instead of 4).
  float* const Cs = smem;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    Cs[(wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * LC + wn * 32 + (lane & 31)] = acc[r];
  __syncthreads();
  const bool cvec = (reinterpret_cast<uintptr_t>(C) & 15) == 0 && a.cmap.s1 % 4 == 0 &&
                    (a.cmap.div == 1 || a.cmap.s2 % 4 == 0);
#pragma unroll
  for (int it = 0; it < BM * BN / 1024; ++it) {
    const int idx = (it * 256 + tid) * 4;
    const int row = idx / BN, col = idx % BN;
    const int m = m0 + row, n = n0 + col;
    if (m >= a.M) continue;
    const float4 cv = *reinterpret_cast<const float4*>(Cs + row * LC + col);
    const float v[4] = {cv.x, cv.y, cv.z, cv.w};
    float* p = C + rowoff(a.cmap, m) + n;
    if (cvec && n + 3 < a.N) {
      float4 o = cv;
      if (a.beta) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        o.x += q.x;
        o.y += q.y;
        o.z += q.z;
        o.w += q.w;
      }
      *reinterpret_cast<float4*>(p) = o;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (n + c < a.N) p[c] = a.beta ? (p[c] + v[c]) : v[c];
    }
  }
}

// ---------------------------------------------------------------- bf16 / fp16 operands
// The reduced-precision option (the analogue of the TF32 channel GEMMs the Sobek paper
// lists as optional in Sec. 4): A and B are read as fp32, rounded to bf16 or fp16
// (nearest, ties to even) when staged in LDS, multiplied on v_mfma_f32_32x32x16_bf16 or
// _f16 and accumulated in fp32.  Tiles as in the fp32 kernels (WGM x WGN wavefronts of
// 32 x 32); LDS holds A as [m][k] and B as [n][k] so each lane reads its eight
// consecutive k as one 16-byte load.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);   // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// F16: fp16 operands (the hardware conversion rounds to nearest, ties to even), else bf16.
template <bool F16>
__device__ inline uint16_t to_low(float f) {
  if constexpr (F16)
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  else
    return bf16_rne(f);
}

template <bool F16>
__device__ inline f16v mfma_low(const uint16_t* a, const uint16_t* b, const f16v& acc) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8*>(a),
                                                  *reinterpret_cast<const f16x8*>(b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a),
                                                   *reinterpret_cast<const bf16x8*>(b), acc, 0, 0, 0);
}

template <int WGM, int WGN, bool F16>
__global__ __launch_bounds__(256) void gemm_low_kernel(const GemmArgs a) {
  constexpr int BM = 32 * WGM, BN = 32 * WGN;
  constexpr int AG = BM / 32, BG = BN / 32;
  constexpr int LK = BK + 8;   // padded k stride (elements): rows stay 16-byte aligned
  __shared__ __attribute__((aligned(16))) uint16_t As[BM][LK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN][LK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid % WGM, wn = wid / WGM;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  const int kz0 = blockIdx.z * a.k_split;
  const int kz1 = min(a.K, kz0 + a.k_split);
  float* C = a.C + static_cast<int64_t>(blockIdx.z) * a.c_split_stride;
  const bool vec = a.vec4 != 0;

  int64_t a_off[AG];
  bool a_ok[AG];
  if (!a.a_mcontig) {
#pragma unroll
    for (int h = 0; h < AG; ++h) {
      const int m = m0 + ((tid + 256 * h) >> 3);
      a_ok[h] = m < a.M;
      a_off[h] = a_ok[h] ? rowoff(a.amap, m) : 0;
    }
  }
  float ra[AG][4], rb[BG][4];
  auto load4 = [&](const float* p, int valid, float* dst) {
    if (valid == 4 && vec) {
      const float4 v = *reinterpret_cast<const float4*>(p);
      dst[0] = v.x;
      dst[1] = v.y;
      dst[2] = v.z;
      dst[3] = v.w;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) dst[t] = t < valid ? p[t] : 0.f;
    }
  };
  auto load = [&](int k0) {
#pragma unroll
    for (int h = 0; h < AG; ++h) {
      const int g = tid + 256 * h;
      if (!a.a_mcontig) {
        const int k = k0 + (g & 7) * 4;
        load4(a.A + a_off[h] + k, a_ok[h] ? min(4, kz1 - k) : 0, ra[h]);
      } else {
        const int k = k0 + g / (BM / 4);
        const int m = m0 + (g % (BM / 4)) * 4;
        const int valid = k < kz1 ? min(4, a.M - m) : 0;
        load4(a.A + (valid > 0 ? rowoff(a.amap, k) : 0) + m, valid, ra[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < BG; ++h) {
      const int g = tid + 256 * h;
      const int k = k0 + g / (BN / 4);
      const int n = n0 + (g % (BN / 4)) * 4;
      const int valid = k < kz1 ? min(4, a.N - n) : 0;
      load4(a.B + static_cast<int64_t>(k < kz1 ? k : 0) * a.ldb + n, valid, rb[h]);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int h = 0; h < AG; ++h) {
      const int g = tid + 256 * h;
      if (!a.a_mcontig) {
        const int row = g >> 3, k4 = (g & 7) * 4;
        const uint32_t lo = to_low<F16>(ra[h][0]) | (static_cast<uint32_t>(to_low<F16>(ra[h][1])) << 16);
        const uint32_t hi = to_low<F16>(ra[h][2]) | (static_cast<uint32_t>(to_low<F16>(ra[h][3])) << 16);
        *reinterpret_cast<uint2*>(&As[row][k4]) = make_uint2(lo, hi);
      } else {
        const int k = g / (BM / 4), m4 = (g % (BM / 4)) * 4;
#pragma unroll
        for (int t = 0; t < 4; ++t) As[m4 + t][k] = to_low<F16>(ra[h][t]);
      }
    }
#pragma unroll
    for (int h = 0; h < BG; ++h) {
      const int g = tid + 256 * h;
      const int k = g / (BN / 4), n4 = (g % (BN / 4)) * 4;
#pragma unroll
      for (int t = 0; t < 4; ++t) Bs[n4 + t][k] = to_low<F16>(rb[h][t]);
    }
  };

  f16v acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (kz0 < kz1) load(kz0);
  // lane l supplies row (or column) l % 32 and the eight k values 8 (l / 32) .. + 7
  const int am = wm * 32 + (lane & 31), bn = wn * 32 + (lane & 31), k8 = 8 * (lane >> 5);
  for (int k0 = kz0; k0 < kz1; k0 += BK) {
    store();
    __syncthreads();
    if (k0 + BK < kz1) load(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      acc = mfma_low<F16>(&As[am][kk + k8], &Bs[bn][kk + k8], acc);
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

// C(m, n) (+)= sum_s part[s][m][n], fixed order in s
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N, float* __restrict__ C,
                                     RowMap cmap, int beta) {
  const int64_t total = static_cast<int64_t>(M) * N;
  for (int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += part[z * total + idx];
    const int m = static_cast<int>(idx / N);
    const int n = static_cast<int>(idx - static_cast<int64_t>(m) * N);
    float* p = C + rowoff(cmap, m) + n;
    *p = beta ? (*p + s) : s;
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int splits, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.lowp) {
    const bool f16 = a.lowp == 2;
    dim3 grid;
    if (a.N <= 32 && a.M > 32) {
      grid = dim3((a.M + 127) / 128, (a.N + 31) / 32, splits);
      if (f16)
        hipLaunchKernelGGL((gemm_low_kernel<4, 1, true>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_low_kernel<4, 1, false>), grid, dim3(256), 0, s, a);
    } else if (a.M <= 32 && a.N > 32) {
      grid = dim3((a.M + 31) / 32, (a.N + 127) / 128, splits);
      if (f16)
        hipLaunchKernelGGL((gemm_low_kernel<1, 4, true>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_low_kernel<1, 4, false>), grid, dim3(256), 0, s, a);
    } else {
      grid = dim3((a.M + 63) / 64, (a.N + 63) / 64, splits);
      if (f16)
        hipLaunchKernelGGL((gemm_low_kernel<2, 2, true>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_low_kernel<2, 2, false>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  // a side of at most 32 (a 32-channel operand) gets a 32-wide tile, so no half tile of
  // MFMA work and loads is wasted on padding
  const bool mc = a.a_mcontig != 0;
  if (a.N <= 32 && a.M > 32) {
    dim3 grid((a.M + 127) / 128, (a.N + 31) / 32, splits);
    if (mc)
      hipLaunchKernelGGL((gemm_f32_kernel<4, 1, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_f32_kernel<4, 1, false>), grid, dim3(256), 0, s, a);
  } else if (a.M <= 32 && a.N > 32) {
    dim3 grid((a.M + 31) / 32, (a.N + 127) / 128, splits);
    if (mc)
      hipLaunchKernelGGL((gemm_f32_kernel<1, 4, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_f32_kernel<1, 4, false>), grid, dim3(256), 0, s, a);
  } else {
    dim3 grid((a.M + 63) / 64, (a.N + 63) / 64, splits);
    if (mc)
      hipLaunchKernelGGL((gemm_f32_kernel<2, 2, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_f32_kernel<2, 2, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int splits, int M, int N, float* C, RowMap cmap, bool beta,
                                hipStream_t s) {
  const int64_t total = static_cast<int64_t>(M) * N;
  if (total <= 0) return hipSuccess;
  int64_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>(g)), dim3(256), 0, s, part, splits, M, N, C,
                     cmap, beta ? 1 : 0);
  return hipGetLastError();
}

}  // namespace etpc
