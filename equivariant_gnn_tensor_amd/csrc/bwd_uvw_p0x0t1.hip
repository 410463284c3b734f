// Instantiation unit: uvw sender traversal, need_p=false pos=false tangent=true.
#include "bwd_impl.hpp"

namespace etpc {
namespace bwd_detail {
template hipError_t launch_bwd_uvw_t<false, false, true, false>(const BwdUvwArgs&, int, int, int, int, hipStream_t);
}  // namespace bwd_detail
}  // namespace etpc
