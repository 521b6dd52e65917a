// ssd_kernels_f16_blk.hip -- the block form (convolution before and norm after the SSD in one
// launch) for f16 inputs, every chunk size.
#include "ssd_kernels.h"

namespace ssd {

hipError_t launch_block_f16(int step, int P, int N, int Q, SsdArgs& a, hipStream_t st) {
    switch (Q) {
    case 64: return dispatch_blk16<_Float16, 64>(step, P, N, a, st);
    case 128: return dispatch_blk16<_Float16, 128>(step, P, N, a, st);
    case 256: return dispatch_blk16<_Float16, 256>(step, P, N, a, st);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ssd
