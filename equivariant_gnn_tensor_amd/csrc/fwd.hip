// Forward launch dispatch (tangent / plain); kernels live in fwd_impl.hpp.
#include "kernels.hpp"

namespace etpc {
namespace fwd_detail {
template <bool T>
hipError_t launch_fwd_uvw_t(const FwdUvwArgs& a, int li, int lo, int nrecv, int ntiles, hipStream_t s);
template <bool T>
hipError_t launch_fwd_uvu_t(const FwdUvuArgs& a, int li, int lo, int n, int ntiles, hipStream_t s);
}  // namespace fwd_detail

hipError_t launch_fwd_uvw(const FwdUvwArgs& a, bool tangent, int li, int lo, int nrecv, int ntiles, hipStream_t s) {
  if (nrecv <= 0) return hipSuccess;
  return tangent ? fwd_detail::launch_fwd_uvw_t<true>(a, li, lo, nrecv, ntiles, s)
                 : fwd_detail::launch_fwd_uvw_t<false>(a, li, lo, nrecv, ntiles, s);
}

hipError_t launch_fwd_uvu(const FwdUvuArgs& a, bool tangent, int li, int lo, int n, int ntiles, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return tangent ? fwd_detail::launch_fwd_uvu_t<true>(a, li, lo, n, ntiles, s)
                 : fwd_detail::launch_fwd_uvu_t<false>(a, li, lo, n, ntiles, s);
}

}  // namespace etpc
