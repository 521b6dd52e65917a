// ssd_kernels_bf16_q256_vl.hip -- kernel instantiations for bf16 inputs, chunk size 256, packed variable-length input (with or without per-sequence states).
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_bf16_q256_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return a.seqstates ? dispatch16<__bf16, 256, 2>(step, P, N, a, st) : dispatch16<__bf16, 256, 1>(step, P, N, a, st);
}

}  // namespace ssd
