// ssd_kernels_f16_q64.hip -- kernel instantiations for f16 inputs, chunk size 64, plain input.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_f16_q64_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return dispatch16<_Float16, 64, 0>(step, P, N, a, st);
}

}  // namespace ssd
