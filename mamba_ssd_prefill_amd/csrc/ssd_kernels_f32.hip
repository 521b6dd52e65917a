// ssd_kernels_f32.hip -- kernel instantiations for f32 inputs.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_f32(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    if (P == 16 && N == 16) return launch_step_t<float, 16, 16>(step, a, st);
    if (P == 16 && N == 32) return launch_step_t<float, 16, 32>(step, a, st);
    if (P == 16 && N == 64) return launch_step_t<float, 16, 64>(step, a, st);
    if (P == 16 && N == 128) return launch_step_t<float, 16, 128>(step, a, st);
    if (P == 32 && N == 16) return launch_step_t<float, 32, 16>(step, a, st);
    if (P == 32 && N == 32) return launch_step_t<float, 32, 32>(step, a, st);
    if (P == 32 && N == 64) return launch_step_t<float, 32, 64>(step, a, st);
    if (P == 32 && N == 128) return launch_step_t<float, 32, 128>(step, a, st);
    if (P == 64 && N == 16) return launch_step_t<float, 64, 16>(step, a, st);
    if (P == 64 && N == 32) return launch_step_t<float, 64, 32>(step, a, st);
    if (P == 64 && N == 64) return launch_step_t<float, 64, 64>(step, a, st);
    if (P == 64 && N == 128) return launch_step_t<float, 64, 128>(step, a, st);
    if (P == 128 && N == 16) return launch_step_t<float, 128, 16>(step, a, st);
    if (P == 128 && N == 32) return launch_step_t<float, 128, 32>(step, a, st);
    if (P == 128 && N == 64) return launch_step_t<float, 128, 64>(step, a, st);
    if (P == 128 && N == 128) return launch_step_t<float, 128, 128>(step, a, st);
    return hipErrorNotSupported;
}

}  // namespace ssd
