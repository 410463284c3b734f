// Shared host/device definitions for the etpc library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <string>

#include "../../include/etpc.h"

namespace etpc {

constexpr int kMaxL = 3;
constexpr int kMaxBasis = 16;
constexpr int kMaxPaths = 64;
constexpr int kWave = 64;

// Concurrent launch lanes of a pass (side streams per device).  Two measured best on
// MI355X: one launch's tail filled by the next; more lanes contend for the four hardware
// queues of a process.  A plan selects 1..kLanes (etpc_spec.lanes).
#ifndef ETPC_LANES
#define ETPC_LANES 2
#endif
constexpr int kLanes = ETPC_LANES;

// Row offset map: row r of a logical matrix lives at (r / div) * s1 + (r % div) * s2.
// Covers plain row-major matrices (div = 1) and ir_mul blocks, whose rows are
// (node, m) pairs: node stride = feature width, m stride = multiplicity.
struct RowMap {
  int64_t s1;
  int64_t s2;
  int32_t div;
  uint32_t magic;   // r / div = (umulhi(r, magic) + r) >> shift for 0 <= r < 2^31
  int32_t shift;
};

// Row map for row r = (r / div, r % div) -> (r / div) * s1 + (r % div) * s2, with the
// division by an invariant integer done as a multiply-high (round-up method: shift =
// ceil(log2 div), magic = floor(2^32 (2^shift - div) / div) + 1).
inline RowMap make_rowmap(int64_t s1, int64_t s2, int32_t div) {
  int32_t l = 0;
  while ((int64_t{1} << l) < div) ++l;
  const uint64_t magic = ((uint64_t{1} << 32) * ((uint64_t{1} << l) - static_cast<uint64_t>(div))) /
                             static_cast<uint64_t>(div) + 1;
  return RowMap{s1, s2, div, static_cast<uint32_t>(magic), l};
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.  The
// receiver traversals take node slot node_block(b, g) for workgroup b of a grid of g, so
// the workgroups of one XCD cover one contiguous range of receivers: with a spatially
// ordered numbering, receivers that share senders then share an L2 (uvu forward -4.5%
// on a Morton-ordered graph, neutral on a random numbering).  The sender traversals
// measured slower with it and keep the plain order.  A bijection on [0, g).
constexpr int kXcds = 8;
__device__ inline int node_block(int b, int g) {
  const int x = b % kXcds, q = g / kXcds, r = g % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

// Edge geometry parameters shared by every traversal kernel.
struct GeomParams {
  int32_t radial;     // etpc_radial
  int32_t nb;         // number of radial bases B
  float r_lo, r_hi;
  float gauss_d;      // Gaussian spacing D
  float gauss_inv2d2; // 1 / (2 D^2)
  int32_t poly_p;
  int32_t periodic;
  float box[3];
  float inv_box[3];
};

// Dense real coupling tensor of one path, stored [NI][7][NO] (m_sh stride fixed at 7).
struct CGTable {
  float c[7 * 7 * 7];
};

}  // namespace etpc

// thread-local error message used by the C ABI
namespace etpc {
void set_error(const std::string& msg);
const char* last_error();
}  // namespace etpc

#define ETPC_FAIL(code, msg)         \
  do {                               \
    ::etpc::set_error(msg);          \
    return (code);                   \
  } while (0)

#define ETPC_HIP(call)                                                                      \
  do {                                                                                      \
    hipError_t _e = (call);                                                                 \
    if (_e != hipSuccess) {                                                                 \
      ::etpc::set_error(std::string("HIP error: ") + hipGetErrorString(_e) + " at " #call); \
      return ETPC_ERR_HIP;                                                                  \
    }                                                                                       \
  } while (0)
