// ssd_kernels_bf16_q256_vl.hip -- kernel instantiations for bf16 inputs, chunk size 256, packed variable-length input.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_bf16_q256_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return dispatch16<__bf16, 256, true>(step, P, N, a, st);
}

}  // namespace ssd
