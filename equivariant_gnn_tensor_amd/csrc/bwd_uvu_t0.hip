// Instantiation unit: uvu sender traversal, tangent=false.
#include "bwd_impl.hpp"

namespace etpc {
namespace bwd_detail {
template hipError_t launch_bwd_uvu_t<false, false>(const BwdUvuArgs&, int, int, int, int, hipStream_t);
}  // namespace bwd_detail
}  // namespace etpc
