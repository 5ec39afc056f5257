// Stand-alone expert-bias update / MaxVio launch: one workgroup of one wave.  The arithmetic
// (and its citations) lives in balance_wave.hpp, which the dispatch scan also runs as an extra
// workgroup when a routed step asks for the update.
#include "balance_wave.hpp"

namespace elb {
namespace {

__global__ __launch_bounds__(64) void balance_kernel(BalanceArgs a) { balance_wave(a); }

}  // namespace

hipError_t launch_balance(const BalanceArgs& a, hipStream_t stream) {
  return launch(balance_kernel, dim3(1), dim3(64), 0, stream, a);
}

}  // namespace elb
