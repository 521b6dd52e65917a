// ssd_kernels_bf16.hip -- bf16 inputs: dispatch on the chunk size.
#include "ssd_launch.h"

namespace ssd {

hipError_t launch_step_bf16(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    switch (a.chunk) {
    case 64: return launch_step_bf16_q64(step, P, N, a, st);
    case 128: return launch_step_bf16_q128(step, P, N, a, st);
    case 256: return launch_step_bf16_q256(step, P, N, a, st);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ssd
