#include "device_common.h"
#include "pkv_internal.h"
namespace pkv {
hipError_t launch_decode_fp8(const DecodeArgs&, int, int64_t, int32_t, hipStream_t) { return hipErrorNotSupported; }
}
