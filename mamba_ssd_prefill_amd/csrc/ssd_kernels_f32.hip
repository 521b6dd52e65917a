// ssd_kernels_f32.hip -- kernel instantiations for f32 inputs (any supported chunk size), plain input.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_f32_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return dispatch32<0>(step, P, N, a, st);
}

hipError_t launch_step_f32(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return a.seq_idx ? launch_step_f32_vl1(step, P, N, a, st) : launch_step_f32_vl0(step, P, N, a, st);
}

}  // namespace ssd
