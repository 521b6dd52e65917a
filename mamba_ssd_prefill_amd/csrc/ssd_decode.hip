// ssd_decode.hip -- one autoregressive step of the SSD recurrence on a cached state.
//
// "Mamba-2状态空间模型的编译器优化与实现", section 2.1 (the O(1) state update: the cache keeps
// the [B,H,P,N] SSM state and each new token applies the recurrence once) and section 3.2
// (decoding is bound by memory bandwidth; all the element-wise work goes into a single pass
// over HBM).  For every batch row b and head h (group g = h / (H / G)):
//
//     dt = softplus(dt_raw[b,h] + dt_bias[h])              (dt_softplus = 1)
//     S  = exp(dt * A[h]) * S + dt * x[b,h,:] (outer) B[b,g,:]
//     y[b,h,:] = S . C[b,g,:] + D[h] * x[b,h,:]
//
// The state dominates the traffic: it is read once and written once, in the state dtype,
// and everything else (x, dt, B, C, y) is a few bytes per row.  So each lane owns four
// consecutive n of one state row and a wave streams whole rows: for N = 128 and an fp32
// state a wave moves 1 KB per load (two rows), and a workgroup issues every load of its rows
// before the first product, which keeps enough bytes in flight to cover the HBM latency.
// The N / 4 lanes of a row reduce y with cross-lane shuffles.  The update is in fp32; the
// state is rounded to its dtype once per step.
#include "ssd_device.h"

namespace ssd {

template <typename S> struct StateIO;
template <> struct StateIO<float> {
    __device__ static inline f32x4 load(const void* base, size_t off) { return *(const f32x4*)((const float*)base + off); }
    __device__ static inline void store(void* base, size_t off, f32x4 v) {
        *(f32x4*)((float*)base + off) = v;
    }
};
template <> struct StateIO<_Float16> {
    __device__ static inline f32x4 load(const void* base, size_t off) {
        const f16x4 v = *(const f16x4*)((const _Float16*)base + off);
        return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
    __device__ static inline void store(void* base, size_t off, f32x4 v) {
        const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        *(f16x4*)((_Float16*)base + off) = h;
    }
};
template <> struct StateIO<__bf16> {
    __device__ static inline f32x4 load(const void* base, size_t off) {
        const bf16x4 v = *(const bf16x4*)((const __bf16*)base + off);
        return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
    __device__ static inline void store(void* base, size_t off, f32x4 v) {
        const bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *(bf16x4*)((__bf16*)base + off) = h;
    }
};

template <typename T> __device__ inline f32x4 load4(const T* p) {
    if constexpr (sizeof(T) == 4) {
        return *(const f32x4*)p;
    } else {
        const typename TT<T>::v4 v = *(const typename TT<T>::v4*)p;
        return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
}

// Workgroup (256 threads) -> (b, h, block of RB = decode_rows_per_block(N) rows of P).
// Wave w, load k covers the RPW = 256 / N consecutive rows starting at
// row0 + (k * 4 + w) * RPW; lane l takes row + l / (N / 4), columns 4 (l % (N / 4)) .. +3.
template <typename T, typename S, int N>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs a) {
    constexpr int LPR = N / 4;      // lanes per state row
    constexpr int RPW = 64 / LPR;   // rows per wave and load
    constexpr int RB = 4 * kDecodeIter * RPW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nblk = (a.headdim + RB - 1) / RB;
    const int pb = blockIdx.x % nblk, h = (blockIdx.x / nblk) % a.nheads, b = blockIdx.x / (nblk * a.nheads);
    const int P = a.headdim, H = a.nheads;
    const int g = h / (H / a.ngroups);
    const int n0 = 4 * (lane % LPR);

    const size_t bh = (size_t)b * H + h;
    const size_t srow0 = bh * P;  // state row index of (b, h, p = 0)
    int rows[kDecodeIter];
    f32x4 s[kDecodeIter];
#pragma unroll
    for (int k = 0; k < kDecodeIter; ++k) {
        rows[k] = pb * RB + (k * 4 + wave) * RPW + lane / LPR;
        s[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.state_in && rows[k] < P) s[k] = StateIO<S>::load(a.state_in, (srow0 + rows[k]) * N + n0);
    }
    const size_t bg = (size_t)b * a.ngroups + g;
    const f32x4 Bv = load4<T>((const T*)a.B + bg * N + n0);
    const f32x4 Cv = load4<T>((const T*)a.C + bg * N + n0);
    float xv[kDecodeIter];
#pragma unroll
    for (int k = 0; k < kDecodeIter; ++k) xv[k] = rows[k] < P ? f32of(((const T*)a.x)[bh * P + rows[k]]) : 0.f;

    const float z = f32of(((const T*)a.dt)[bh]) + (a.dt_bias ? a.dt_bias[h] : 0.f);
    const float dt = a.softplus ? softplus_f(z) : z;
    const float dec = __expf(dt * a.A[h]);
    const float Dh = a.D ? a.D[h] : 0.f;

#pragma unroll
    for (int k = 0; k < kDecodeIter; ++k) {
        const float u = dt * xv[k];
        f32x4 sn;
#pragma unroll
        for (int e = 0; e < 4; ++e) sn[e] = dec * s[k][e] + u * Bv[e];
        float yp = sn[0] * Cv[0] + sn[1] * Cv[1] + sn[2] * Cv[2] + sn[3] * Cv[3];
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) yp += __shfl_xor(yp, m, 64);
        if (rows[k] < P) {
            StateIO<S>::store(a.state_out, (srow0 + rows[k]) * N + n0, sn);
            if (lane % LPR == 0) ((T*)a.y)[bh * P + rows[k]] = (T)(yp + Dh * xv[k]);
        }
    }
}

template <typename T, typename S> hipError_t launch_decode_ts(DecodeArgs& a, hipStream_t st) {
    const void* fn = nullptr;
    switch (a.dstate) {
    case 16: fn = (const void*)&k_decode<T, S, 16>; break;
    case 32: fn = (const void*)&k_decode<T, S, 32>; break;
    case 64: fn = (const void*)&k_decode<T, S, 64>; break;
    case 128: fn = (const void*)&k_decode<T, S, 128>; break;
    case 256: fn = (const void*)&k_decode<T, S, 256>; break;
    default: return hipErrorNotSupported;
    }
    const int rb = decode_rows_per_block(a.dstate);
    const unsigned nblk = (unsigned)((a.headdim + rb - 1) / rb);
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3(nblk * (unsigned)a.nheads * (unsigned)a.batch), dim3(256), args, 0, st);
}

template <typename T> hipError_t launch_decode_t(DecodeArgs& a, hipStream_t st) {
    switch (a.state_dtype) {
    case DT_F32: return launch_decode_ts<T, float>(a, st);
    case DT_F16: return launch_decode_ts<T, _Float16>(a, st);
    case DT_BF16: return launch_decode_ts<T, __bf16>(a, st);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_decode(DecodeArgs& a, int in_dtype, hipStream_t st) {
    switch (in_dtype) {
    case DT_F32: return launch_decode_t<float>(a, st);
    case DT_F16: return launch_decode_t<_Float16>(a, st);
    case DT_BF16: return launch_decode_t<__bf16>(a, st);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ssd
