// ssd_kernels_f16_q256.hip -- kernel instantiations for f16 inputs, chunk size 256, plain input.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_f16_q256_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return dispatch16<_Float16, 256, 0>(step, P, N, a, st);
}

}  // namespace ssd
