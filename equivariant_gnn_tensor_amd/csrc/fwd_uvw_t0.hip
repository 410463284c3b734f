// Instantiation unit: uvw forward traversal, tangent=false.
#include "fwd_impl.hpp"

namespace etpc {
namespace fwd_detail {
template hipError_t launch_fwd_uvw_t<false>(const FwdUvwArgs&, int, int, int, int, hipStream_t);
}  // namespace fwd_detail
}  // namespace etpc
