// ssd_kernels_bf16_q128_vl.hip -- kernel instantiations for bf16 inputs, chunk size 128, packed variable-length input (with or without per-sequence states).
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_bf16_q128_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return a.seqstates ? dispatch16<__bf16, 128, 2>(step, P, N, a, st) : dispatch16<__bf16, 128, 1>(step, P, N, a, st);
}

}  // namespace ssd
