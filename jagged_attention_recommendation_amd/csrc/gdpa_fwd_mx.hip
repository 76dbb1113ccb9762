// Forward launches for MX-fp8 inputs: e4m3 Q/K/V with e8m0 scales per 32 elements along D
// (kernel template in gdpa_fwd_kernel.h). D = 128 only.
#include "gdpa_fwd_kernel.h"

namespace gdpa {

hipError_t launch_fwd_mx(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (p.D != 128) return hipErrorNotSupported;
  return fwdk::launch_d<128, true>(p, a, grid, s);
}

}  // namespace gdpa
