#include "gdpa_common.h"
#include "gdpa_internal.h"
namespace gdpa {
hipError_t launch_bwd_bf16(const Prob&, const BwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdpa
