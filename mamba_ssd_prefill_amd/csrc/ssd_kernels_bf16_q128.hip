// ssd_kernels_bf16_q128.hip -- kernel instantiations for bf16 inputs, chunk size 128.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_bf16_q128(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    if (P == 16 && N == 32) return launch_step16<__bf16, 16, 32, 128>(step, a, st);
    if (P == 16 && N == 64) return launch_step16<__bf16, 16, 64, 128>(step, a, st);
    if (P == 16 && N == 128) return launch_step16<__bf16, 16, 128, 128>(step, a, st);
    if (P == 32 && N == 32) return launch_step16<__bf16, 32, 32, 128>(step, a, st);
    if (P == 32 && N == 64) return launch_step16<__bf16, 32, 64, 128>(step, a, st);
    if (P == 32 && N == 128) return launch_step16<__bf16, 32, 128, 128>(step, a, st);
    if (P == 64 && N == 32) return launch_step16<__bf16, 64, 32, 128>(step, a, st);
    if (P == 64 && N == 64) return launch_step16<__bf16, 64, 64, 128>(step, a, st);
    if (P == 64 && N == 128) return launch_step16<__bf16, 64, 128, 128>(step, a, st);
    if (P == 128 && N == 32) return launch_step16<__bf16, 128, 32, 128>(step, a, st);
    if (P == 128 && N == 64) return launch_step16<__bf16, 128, 64, 128>(step, a, st);
    if (P == 128 && N == 128) return launch_step16<__bf16, 128, 128, 128>(step, a, st);
    return hipErrorNotSupported;
}

}  // namespace ssd
