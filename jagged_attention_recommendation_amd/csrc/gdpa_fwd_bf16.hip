// Forward launches for bf16 inputs: D = 128 uses the direct-load kernel (gdpa_fwd_dl.h), D = 32
// and 64 the register-staged one (gdpa_fwd_kernel.h).
#include "gdpa_fwd_dl.h"
#include "gdpa_fwd_kernel.h"

namespace gdpa {

hipError_t launch_fwd_bf16(const Prob& p, const FwdArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (p.D) {
    case 32: return fwdk::launch_d<32, false>(p, a, grid, s);
    case 64: return fwdk::launch_d<64, false>(p, a, grid, s);
    default: return fwddl::launch(p, a, grid, s);
  }
}

}  // namespace gdpa
