// ssd_kernels_f32_vl.hip -- kernel instantiations for f32 inputs (any supported chunk size), packed variable-length input.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_f32_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return dispatch32<1>(step, P, N, a, st);
}

}  // namespace ssd
