// ssd_kernels_f16_q256_vl.hip -- kernel instantiations for f16 inputs, chunk size 256, packed variable-length input (with or without per-sequence states).
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_step_f16_q256_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    return a.seqstates ? dispatch16<_Float16, 256, 2>(step, P, N, a, st) : dispatch16<_Float16, 256, 1>(step, P, N, a, st);
}

}  // namespace ssd
