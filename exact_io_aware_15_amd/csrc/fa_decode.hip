#include "fa_kernels.h"
namespace fa355 {
hipError_t launch_decode(const DecodeArgs &, int, hipStream_t) { return hipErrorNotSupported; }
}
