// ssd_kernels_f16_q128.hip -- kernel instantiations for f16 inputs, chunk size 128, plain input.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_f16_q128_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return dispatch16<_Float16, 128, 0>(step, P, N, a, st);
}

}  // namespace ssd
