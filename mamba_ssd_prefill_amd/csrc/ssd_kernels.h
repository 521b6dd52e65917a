// ssd_kernels.h -- __global__ entry points of the SSD prefill and their host launchers.
// Included once per input dtype by ssd_kernels_{f32,f16,bf16}.hip, which instantiate
// the launchers for the supported (headdim, dstate) pairs.
#pragma once

#include "ssd_device.h"
#include "ssd_tile16.h"

namespace ssd {

// ---- unfused form: one kernel per step -------------------------------------------------
template <typename T> __global__ __launch_bounds__(256) void k_chunk_cumsum(SsdArgs a) {
    const int c = blockIdx.x % a.nchunks, b = blockIdx.x / a.nchunks;
    cumsum_tile<T, false>(a, b, c);
}

template <typename T, int N> __global__ __launch_bounds__(256) void k_bmm(SsdArgs a) {
    const int g = blockIdx.x % a.ngroups;
    const int c = (blockIdx.x / a.ngroups) % a.nchunks;
    const int b = blockIdx.x / (a.ngroups * a.nchunks);
    bmm_tile<T, N, false>(a, b, c, g);
}

// blockIdx.x -> (b, c, g, tile-in-group)
template <typename T, int P, int N, int MODE> __global__ __launch_bounds__(256) void k_chunk(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo<T, P, N>::SMEM];
    int r = blockIdx.x;
    const int tig = r % a.tpg;
    r /= a.tpg;
    const int g = r % a.ngroups;
    r /= a.ngroups;
    const int c = r % a.nchunks;
    const int b = r / a.nchunks;
    chunk_tile<T, P, N, MODE>(a, b, c, g, tig, smem);
}

// ---- fused form: a single launch ([KF] "高效内核融合技术揭秘") ------------------------------
// Each workgroup takes one ticket.  Tickets [0, T_cs) are cumsum tiles (b, c) in chunk
// order, [T_cs, T_cs + T_bmm) are bmm tiles (b, c, g) in chunk order, the rest are chunk
// tiles (c, b, g, tile-in-group) in chunk-major order.  A chunk tile waits only on work
// with smaller tickets (its cumsum and bmm tiles and the previous chunk's tile of its
// chains), all of which were claimed by running workgroups, so the waits always end.
template <typename T, int P, int N> __global__ __launch_bounds__(256) void k_fused(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo<T, P, N>::SMEM];
    __shared__ uint32_t s_ticket;
    if (threadIdx.x == 0) s_ticket = atomicAdd(a.ticket, 1u);
    __syncthreads();
    const uint32_t t = __builtin_amdgcn_readfirstlane(s_ticket);  // uniform: keeps tile math scalar
    const uint32_t Bn = a.batch, nc = a.nchunks, Gn = a.ngroups, tpg = a.tpg;
    const uint32_t t_cs = Bn * nc, t_bmm = Bn * nc * Gn;
    if (t >= t_cs + t_bmm + Bn * nc * Gn * tpg) return;  // only if the ticket word was not reset
    if (t < t_cs) {
        const int c = t / Bn, b = t % Bn;
        cumsum_tile<T, true>(a, b, c);
        publish_flag_block(a.cs_done + (size_t)b * nc + c);
    } else if (t < t_cs + t_bmm) {
        const uint32_t u = t - t_cs;
        const int c = u / (Bn * Gn), b = (u / Gn) % Bn, g = u % Gn;
        bmm_tile<T, N, true>(a, b, c, g);
        publish_flag_block(a.bmm_done + ((size_t)b * nc + c) * Gn + g);
    } else {
        const uint32_t u = t - t_cs - t_bmm;
        const uint32_t per_chunk = Bn * Gn * tpg;
        const int c = u / per_chunk;
        const uint32_t rem = u % per_chunk;
        const int b = rem / (Gn * tpg), g = (rem / tpg) % Gn, tig = rem % tpg;
        if (threadIdx.x == 0) {
            wait_flag(a.cs_done + (size_t)b * nc + c, a);
            wait_flag(a.bmm_done + ((size_t)b * nc + c) * Gn + g, a);
        }
        __syncthreads();
        chunk_tile<T, P, N, MODE_FUSED>(a, b, c, g, tig, smem);
    }
}

// ---- 16-bit inputs: chunk tiles with the chunk size fixed at compile time ------------------
template <typename T, int P, int N, int Q, int MODE> __global__ __launch_bounds__(256) void k_chunk16(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo16<T, P, N, Q>::SMEM];
    int r = blockIdx.x;
    const int tig = r % a.tpg;
    r /= a.tpg;
    const int g = r % a.ngroups;
    r /= a.ngroups;
    const int c = r % a.nchunks;
    const int b = r / a.nchunks;
    chunk_tile16<T, P, N, Q, MODE>(a, b, c, g, tig, smem);
}

template <typename T, int P, int N, int Q> __global__ __launch_bounds__(256, 2) void k_fused16(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo16<T, P, N, Q>::SMEM];
    __shared__ uint32_t s_ticket;
    if (threadIdx.x == 0) s_ticket = atomicAdd(a.ticket, 1u);
    __syncthreads();
    const uint32_t t = __builtin_amdgcn_readfirstlane(s_ticket);  // uniform: keeps tile math scalar
    const uint32_t Bn = a.batch, nc = a.nchunks, Gn = a.ngroups, tpg = a.tpg;
    const uint32_t t_cs = Bn * nc, t_bmm = Bn * nc * Gn;
    if (t >= t_cs + t_bmm + Bn * nc * Gn * tpg) return;  // only if the ticket word was not reset
    if (t < t_cs) {
        const int c = t / Bn, b = t % Bn;
        cumsum_tile<T, true>(a, b, c);
        publish_flag_block(a.cs_done + (size_t)b * nc + c);
    } else if (t < t_cs + t_bmm) {
        const uint32_t u = t - t_cs;
        const int c = u / (Bn * Gn), b = (u / Gn) % Bn, g = u % Gn;
        bmm_tile<T, N, true>(a, b, c, g);
        publish_flag_block(a.bmm_done + ((size_t)b * nc + c) * Gn + g);
    } else {
        const uint32_t u = t - t_cs - t_bmm;
        const uint32_t per_chunk = Bn * Gn * tpg;
        const int c = u / per_chunk;
        const uint32_t rem = u % per_chunk;
        const int b = rem / (Gn * tpg), g = (rem / tpg) % Gn, tig = rem % tpg;
        if (threadIdx.x == 0) {
            wait_flag(a.cs_done + (size_t)b * nc + c, a);
            wait_flag(a.bmm_done + ((size_t)b * nc + c) * Gn + g, a);
        }
        __syncthreads();
        chunk_tile16<T, P, N, Q, MODE_FUSED>(a, b, c, g, tig, smem);
    }
}

// ---- host launchers ----------------------------------------------------------------------
inline hipError_t launch(const void* fn, unsigned grid, void* arg0, hipStream_t st) {
    void* args[] = {arg0};
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, st);
}

template <typename T, int P, int N> hipError_t launch_step_t(int step, SsdArgs& a, hipStream_t st) {
    typedef Geo<T, P, N> G_;
    const unsigned Bn = a.batch, nc = a.nchunks, Gn = a.ngroups, tpg = a.tpg;
    switch (step) {
    case STEP_CUMSUM:
        return launch((const void*)&k_chunk_cumsum<T>, Bn * nc, &a, st);
    case STEP_BMM:
        return launch((const void*)&k_bmm<T, N>, Bn * nc * Gn, &a, st);
    case STEP_CHUNK_STATE:
        return launch((const void*)&k_chunk<T, P, N, MODE_STATE>, Bn * nc * Gn * tpg, &a, st);
    case STEP_STATE_PASSING:
        return launch_state_passing(a, P * N, st);
    case STEP_CHUNK_SCAN:
        return launch((const void*)&k_chunk<T, P, N, MODE_SCAN>, Bn * nc * Gn * tpg, &a, st);
    case STEP_FUSED:
        return launch((const void*)&k_fused<T, P, N>, Bn * nc + Bn * nc * Gn + Bn * nc * Gn * tpg, &a, st);
    default:
        return hipErrorInvalidValue;
    }
    (void)sizeof(G_);
}

template <typename T, int P, int N, int Q> hipError_t launch_step16(int step, SsdArgs& a, hipStream_t st) {
    const unsigned Bn = a.batch, nc = a.nchunks, Gn = a.ngroups, tpg = a.tpg;
    switch (step) {
    case STEP_CUMSUM:
        return launch((const void*)&k_chunk_cumsum<T>, Bn * nc, &a, st);
    case STEP_BMM:
        return launch((const void*)&k_bmm<T, N>, Bn * nc * Gn, &a, st);
    case STEP_CHUNK_STATE:
        return launch((const void*)&k_chunk16<T, P, N, Q, MODE_STATE>, Bn * nc * Gn * tpg, &a, st);
    case STEP_STATE_PASSING:
        return launch_state_passing(a, P * N, st);
    case STEP_CHUNK_SCAN:
        return launch((const void*)&k_chunk16<T, P, N, Q, MODE_SCAN>, Bn * nc * Gn * tpg, &a, st);
    case STEP_FUSED:
        return launch((const void*)&k_fused16<T, P, N, Q>, Bn * nc + Bn * nc * Gn + Bn * nc * Gn * tpg, &a, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace ssd
