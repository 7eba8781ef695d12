// forward_gather_split.hip -- the gather kernel instantiated for the balanced
// partition (workgroups over equal ranges of row ends + edges, heavy rows cut
// and merged across workgroups); compiled apart from forward_gather.hip so
// that the two sets of kernels build in parallel.
#include "gather_kernel.hpp"

namespace gattn {
namespace detail {
template <>
int resident_of<kPartSplit>(const Problem& p) { return resident_impl<kPartSplit>(p); }
template <>
hipError_t launch_kernels<kPartSplit>(const Problem& p, const GatherArgs& ga, dim3 grid, hipStream_t s) {
  return launch_impl<kPartSplit>(p, ga, grid, s);
}
}  // namespace detail
}  // namespace gattn
