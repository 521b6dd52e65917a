// ssd_kernels_bf16_q128.hip -- kernel instantiations for bf16 inputs, chunk size 128, plain input.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_bf16_q128_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return dispatch16<__bf16, 128, 0>(step, P, N, a, st);
}

}  // namespace ssd
