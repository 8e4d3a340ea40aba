#include "device_common.h"
#include "kernels.h"
namespace pd {
hipError_t launch_mla_verify(const MlaArgs&, hipStream_t) { return hipErrorNotSupported; }
}
