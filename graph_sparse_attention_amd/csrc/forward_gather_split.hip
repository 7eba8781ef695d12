// forward_gather_split.hip -- the gather kernel instantiated for the balanced
// partition (workgroups over equal ranges of row ends + edges, heavy rows cut
// and merged across workgroups); compiled apart from forward_gather.hip so
// that the two sets of kernels build in parallel.
#include "gather_kernel.hpp"

namespace gattn {
namespace detail {
template <>
int resident_of<true>(const Problem& p) { return resident_impl<true>(p); }
template <>
hipError_t launch_kernels<true>(const Problem& p, const GatherArgs& ga, dim3 grid, hipStream_t s) {
  return launch_impl<true>(p, ga, grid, s);
}
}  // namespace detail
}  // namespace gattn
