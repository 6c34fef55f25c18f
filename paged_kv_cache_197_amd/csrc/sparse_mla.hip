#include "args.hpp"
#include "common.hpp"
#include "launch.hpp"
namespace pkv_launch {
size_t sparse_workspace_bytes(int, int, int, int) { return 0; }
hipError_t sparse_topk(const pkv::SparseArgs&, hipStream_t) { return hipErrorNotSupported; }
}
