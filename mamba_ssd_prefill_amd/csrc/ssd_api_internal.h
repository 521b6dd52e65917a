// ssd_api_internal.h -- library-internal entry shared by the C-ABI translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mamba_ssd.h"

namespace ssd {

// Per-sequence states of packed input (ssd_prefill_varlen_states); all null / 0 otherwise.
struct SeqStates {
    const void* initial;  // [nseq][H][P][N] or nullptr
    void* final_;         // [nseq][H][P][N]; nullptr: not this mode
    int nseq;
};

// ssd_prefill / _varlen / _varlen_states / _timed behind their argument checks (ssd_api.cpp):
// validates *p and every pointer, then enqueues the whole prefill on `stream` using `workspace`.
ssd_status_t prefill_impl(const ssd_params_t* p, const void* x, const void* dt, const float* A, const void* B,
                          const void* C, const float* D, const float* dt_bias, const void* initial_state, void* y,
                          void* final_state, void* workspace, size_t workspace_bytes, void* stream,
                          hipEvent_t ev_begin, hipEvent_t ev_end, const int32_t* seq_idx,
                          const SeqStates& ss = SeqStates{nullptr, nullptr, 0});

}  // namespace ssd
