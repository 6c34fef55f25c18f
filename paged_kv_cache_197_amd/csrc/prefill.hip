#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"
namespace pkv_launch {
hipError_t prefill(const pkv::PrefillArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}
