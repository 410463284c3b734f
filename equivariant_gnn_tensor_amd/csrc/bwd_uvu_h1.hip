// Instantiation unit: uvu sender traversal, position Hessian along pos_dot (double backward).
#include "bwd_impl.hpp"

namespace etpc {
namespace bwd_detail {
template hipError_t launch_bwd_uvu_t<false, true>(const BwdUvuArgs&, int, int, int, int, hipStream_t);
}  // namespace bwd_detail
}  // namespace etpc
