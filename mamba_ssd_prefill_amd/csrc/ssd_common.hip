// ssd_common.hip -- the dtype-independent kernels: state_passing of the unfused form and
// the boundary copies shared by both forms.
#include "ssd_device.h"

namespace ssd {

// state_passing ("Mamba-2炸裂升级！…", section "Mamba-2核心操作与融合的必要性", item 6):
// one thread per 4 consecutive state elements of one (b, h), sequential over the chunks:
// S_{c+1} = exp(acs_c[Q-1]) S_c + s_c, carried in fp32 and stored to slot c + 1 in the
// state dtype (the decay is 0 when a packed sequence starts inside chunk c).  Slot 0 holds
// the initial state (written by the boundary copy).
__global__ __launch_bounds__(256) void k_state_passing(SsdArgs a, int PN) {
    const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= PN) return;
    const int h = blockIdx.y, b = blockIdx.z;
    const int H = a.nheads, nc = a.nchunks, Q = a.chunk, K = a.slots;
    f32x4 S = load_state4(a.states, a.state_dtype, ((size_t)b * K * H + h) * PN + e);
    if (a.seq_idx) {
        // packed input: a sequence that starts inside chunk c passes no state on; with
        // per-sequence states the state passed on carries that sequence's initial state instead,
        // decayed from just before its first token (found by bisecting the start counts) to the
        // chunk end
        for (int c = 0; c < nc; ++c) {
            const int* sg = a.seg + ((size_t)b * nc + c) * Q;
            const float* ac = a.acs + (((size_t)b * nc + c) * H + h) * Q;
            const int kc = sg[Q - 1];
            const float dec = kc != 0 ? 0.f : __expf(ac[Q - 1]);
            const f32x4 sl = *(const f32x4*)(a.s + (((size_t)b * nc + c) * H + h) * PN + e);
            S = dec * S + sl;
            if (a.seqstates && a.seq_h0 && kc != 0) {
                int lo = 0, hi = Q - 1;  // the first token with sg == kc
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (sg[mid] >= kc) hi = mid; else lo = mid + 1;
                }
                const int q = a.seq_idx[(size_t)b * a.seqlen + (size_t)c * Q + lo];
                if (q >= 0 && q < a.nseq)
                    S += __expf(ac[Q - 1] - (lo > 0 ? ac[lo - 1] : 0.f)) *
                         load_state4(a.seq_h0, a.state_dtype, ((size_t)q * H + h) * PN + e);
            }
            store_state4(a.states, a.state_dtype, (((size_t)b * K + c + 1) * H + h) * PN + e, S);
        }
        return;
    }
#pragma unroll 4
    for (int c = 0; c < nc; ++c) {
        const float dec = __expf(a.acs[(((size_t)b * nc + c) * H + h) * Q + Q - 1]);
        const f32x4 sl = *(const f32x4*)(a.s + (((size_t)b * nc + c) * H + h) * PN + e);
        S = dec * S + sl;
        store_state4(a.states, a.state_dtype, (((size_t)b * K + c + 1) * H + h) * PN + e, S);
    }
}

// Boundary copies (same write-up, section "性能瓶颈的深入分析": the initial state goes into
// chunk 0's slot and the final state comes out of the last chunk's slot, outside the
// fused kernel).  Copies bytes_per_b bytes per batch row from src (batch stride src_bs)
// to dst (batch stride dst_bs), 16 bytes per thread; src == nullptr writes zeros.  Also
// resets nsync sync words: word i becomes 1 when i < nflags and i % flag_period == 0
// (chunk 0's flag of every chain: the initial state is ready), else 0.
__global__ __launch_bounds__(256) void k_boundary(const char* src, size_t src_bs, char* dst, size_t dst_bs,
                                                   size_t bytes_per_b, int batch, uint32_t* sync, size_t nsync,
                                                   size_t nflags, uint32_t flag_period) {
    const size_t n16 = bytes_per_b / 16;
    const size_t total = n16 * (size_t)batch;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const size_t b = i / n16, k = i % n16;
        uint4 v = {0u, 0u, 0u, 0u};
        if (src) v = *(const uint4*)(src + b * src_bs + k * 16);
        *(uint4*)(dst + b * dst_bs + k * 16) = v;
    }
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nsync; i += stride)
        sync[i] = (i < nflags && (i % flag_period) == 0) ? 1u : 0u;
}

// Boundary copies of the fused form, between the callers' [B][H][P][N] states and the ring
// layout (see ring_chain): to_ring = 1 copies src into slot `slot`, to_ring = 0
// copies slot `slot` out to dst (src == nullptr: no initial state, nothing is copied).  One
// thread per 4 consecutive n of one (b, h, p).  pperm = 1:
// the 16-bit tile's interleaved p order (Geo16::pcol), else p block pb = pw / 16, lane pw % 16.  Also
// resets nsync sync words, all but word `keep`: word i becomes flag_init when i < nflags and
// i % flag_period < 4 (the progress counters of every chain, one per relay wave: 1 = the state
// entering chunk 0 is ready), else 0.  The final-state copy does this for the next call.
__global__ __launch_bounds__(256) void k_ring_copy(const char* src, char* dst, int to_ring, int B, int H, int P,
                                                    int PW, int N, int K, int slot, int es, int pperm,
                                                    uint32_t* sync, size_t nsync, size_t nflags,
                                                    uint32_t flag_period, uint32_t flag_init, size_t keep) {
    const int WPH = P / PW, MBP = PW / 16, NB = N / 16;
    const int n4 = N / 4, per_bh = P * n4;  // items (4 consecutive n) per (b, h); P, N powers of 2
    const int nsh = __builtin_ctz((unsigned)n4), bsh = __builtin_ctz((unsigned)per_bh);
    // no initial state: the fused kernel never reads slot 0 before writing it, so nothing to copy
    const size_t items = (to_ring && src == nullptr) ? 0 : (size_t)B * H * per_bh;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < items; i += stride) {
        const size_t bh = i >> bsh;
        const int e = (int)(i & (size_t)(per_bh - 1));
        const int b = (int)(bh / (size_t)H), h = (int)(bh - (size_t)b * H);
        const int p = e >> nsh, n = (e & (n4 - 1)) * 4;
        const int ph = p / PW, pw = p - ph * PW;
        int pb = pw >> 4, r16 = pw & 15;
        if (pperm) {
            const int q8 = pw / (4 * MBP), rem = pw - q8 * 4 * MBP;
            pb = rem >> 2;
            r16 = 4 * q8 + (rem & 3);
        }
        const int nb = n >> 4, q = (n & 15) >> 2;
        const size_t ring =
            ring_chain(b, slot, h, ph, K, H, WPH, NB * MBP) + (size_t)(((nb * MBP + pb) * 64 + 16 * q + r16) * 4);
        const size_t user = bh * P * N + (size_t)(p * N + n);
        const size_t from = to_ring ? user : ring, to = to_ring ? ring : user;
        if (es == 4) {
            uint4 v = {0u, 0u, 0u, 0u};
            if (src) v = *(const uint4*)(src + from * 4);
            *(uint4*)(dst + to * 4) = v;
        } else {
            uint2 v = {0u, 0u};
            if (src) v = *(const uint2*)(src + from * 2);
            *(uint2*)(dst + to * 2) = v;
        }
    }
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nsync; i += stride)
        if (i != keep) sync[i] = (i < nflags && (i % flag_period) < 4u) ? flag_init : 0u;
}

hipError_t launch_ring_copy(const void* src, void* dst, int to_ring, int B, int H, int P, int PW, int N, int K,
                            int slot, int es, int pperm, uint32_t* sync, size_t nsync, size_t nflags,
                            uint32_t flag_period, uint32_t flag_init, size_t keep, hipStream_t st) {
    const size_t items = (to_ring && src == nullptr) ? 0 : (size_t)B * H * P * (N / 4);
    const size_t big = items > nsync ? items : nsync;
    size_t grid = (big + 255) / 256;
    if (grid < 1) grid = 1;
    if (grid > 8192) grid = 8192;
    const char* s = (const char*)src;
    char* d = (char*)dst;
    void* args[] = {&s, &d, &to_ring, &B, &H, &P, &PW, &N, &K, &slot, &es, &pperm, &sync, &nsync, &nflags,
                    &flag_period, &flag_init, &keep};
    return hipLaunchKernel((const void*)&k_ring_copy, dim3((unsigned)grid), dim3(256), args, 0, st);
}

hipError_t launch_state_passing(SsdArgs& a, int PN, hipStream_t st) {
    void* args[] = {&a, &PN};
    return hipLaunchKernel((const void*)&k_state_passing, dim3((PN / 4 + 255) / 256, a.nheads, a.batch),
                           dim3(256), args, 0, st);
}

hipError_t launch_boundary(const void* src, size_t src_bs, void* dst, size_t dst_bs, size_t bytes_per_b,
                           int batch, uint32_t* sync, size_t nsync, size_t nflags, uint32_t flag_period,
                           hipStream_t st) {
    const size_t work = (bytes_per_b / 16) * (size_t)batch;
    const size_t big = work > nsync ? work : nsync;
    size_t grid = (big + 255) / 256;
    if (grid < 1) grid = 1;
    if (grid > 4096) grid = 4096;
    const char* s = (const char*)src;
    char* d = (char*)dst;
    void* args[] = {&s, &src_bs, &d, &dst_bs, &bytes_per_b, &batch, &sync, &nsync, &nflags, &flag_period};
    return hipLaunchKernel((const void*)&k_boundary, dim3((unsigned)grid), dim3(256), args, 0, st);
}

}  // namespace ssd
