// Backward launch dispatch; kernels live in bwd_impl.hpp.
#include "kernels.hpp"

namespace etpc {
namespace bwd_detail {
template <bool NEED_P, bool POS, bool TAN, bool HESS>
hipError_t launch_bwd_uvw_t(const BwdUvwArgs& a, int li, int lo, int nsend, int ntiles, hipStream_t s);
template <bool TAN, bool HESS>
hipError_t launch_bwd_uvu_t(const BwdUvuArgs& a, int li, int lo, int nblocks, int ntiles, hipStream_t s);
}  // namespace bwd_detail

hipError_t launch_bwd_uvw(const BwdUvwArgs& a, bool need_p, bool need_pos, bool tangent, bool hess, int li, int lo,
                          int nsend, int ntiles, hipStream_t s) {
  if (nsend <= 0) return hipSuccess;
  if (hess) {
    if (need_p || !need_pos || tangent) return hipErrorInvalidValue;
    return bwd_detail::launch_bwd_uvw_t<false, true, false, true>(a, li, lo, nsend, ntiles, s);
  }
  if (need_p == true && need_pos == false && tangent == false)
    return bwd_detail::launch_bwd_uvw_t<true, false, false, false>(a, li, lo, nsend, ntiles, s);
  if (need_p == true && need_pos == true && tangent == false)
    return bwd_detail::launch_bwd_uvw_t<true, true, false, false>(a, li, lo, nsend, ntiles, s);
  if (need_p == false && need_pos == true && tangent == false)
    return bwd_detail::launch_bwd_uvw_t<false, true, false, false>(a, li, lo, nsend, ntiles, s);
  if (need_p == false && need_pos == false && tangent == true)
    return bwd_detail::launch_bwd_uvw_t<false, false, true, false>(a, li, lo, nsend, ntiles, s);
  if (need_p == true && need_pos == false && tangent == true)
    return bwd_detail::launch_bwd_uvw_t<true, false, true, false>(a, li, lo, nsend, ntiles, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_uvu(const BwdUvuArgs& a, bool tangent, bool hess, int li, int lo, int nblocks, int ntiles,
                          hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  if (hess) {
    if (tangent) return hipErrorInvalidValue;
    return bwd_detail::launch_bwd_uvu_t<false, true>(a, li, lo, nblocks, ntiles, s);
  }
  return tangent ? bwd_detail::launch_bwd_uvu_t<true, false>(a, li, lo, nblocks, ntiles, s)
                 : bwd_detail::launch_bwd_uvu_t<false, false>(a, li, lo, nblocks, ntiles, s);
}

}  // namespace etpc
