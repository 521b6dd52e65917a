// ssd_kernels_bf16_q256.hip -- kernel instantiations for bf16 inputs, chunk size 256, plain input.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_bf16_q256_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return dispatch16<__bf16, 256, 0>(step, P, N, a, st);
}

}  // namespace ssd
