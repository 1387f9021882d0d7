#include "device_common.h"
#include "pkv_internal.h"
namespace pkv {
hipError_t launch_extend_bf16(const ExtendArgs&, int, int64_t, hipStream_t) { return hipErrorNotSupported; }
}
