// Instantiation unit: uvw sender traversal, position Hessian along pos_dot (double backward).
#include "bwd_impl.hpp"

namespace etpc {
namespace bwd_detail {
template hipError_t launch_bwd_uvw_t<false, true, false, true>(const BwdUvwArgs&, int, int, int, int, hipStream_t);
}  // namespace bwd_detail
}  // namespace etpc
