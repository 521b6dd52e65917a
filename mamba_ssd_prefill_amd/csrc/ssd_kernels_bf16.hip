// ssd_kernels_bf16.hip -- bf16 inputs: dispatch on the chunk size and on packed input.
#include "ssd_launch.h"

namespace ssd {

hipError_t launch_step_bf16(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    const bool vl = a.seq_idx != nullptr;
    switch (a.chunk) {
    case 64: return vl ? launch_step_bf16_q64_vl1(step, P, N, a, st) : launch_step_bf16_q64_vl0(step, P, N, a, st);
    case 128: return vl ? launch_step_bf16_q128_vl1(step, P, N, a, st) : launch_step_bf16_q128_vl0(step, P, N, a, st);
    case 256: return vl ? launch_step_bf16_q256_vl1(step, P, N, a, st) : launch_step_bf16_q256_vl0(step, P, N, a, st);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ssd
