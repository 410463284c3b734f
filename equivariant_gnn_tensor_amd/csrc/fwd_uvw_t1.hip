// Instantiation unit: uvw forward traversal, tangent=true.
#include "fwd_impl.hpp"

namespace etpc {
namespace fwd_detail {
template hipError_t launch_fwd_uvw_t<true>(const FwdUvwArgs&, int, int, int, int, hipStream_t);
}  // namespace fwd_detail
}  // namespace etpc
