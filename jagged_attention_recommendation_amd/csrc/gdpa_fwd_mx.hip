#include "gdpa_common.h"
#include "gdpa_internal.h"
namespace gdpa {
hipError_t launch_fwd_mx(const Prob&, const FwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdpa
