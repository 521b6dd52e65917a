// ssd_block.hip -- the steps around the SSD in the Mamba-2 block, as separate kernels: the
// causal depthwise convolution with SiLU before it and the gated RMS norm after it
// ("Mamba-2炸裂升级！…", section "未来展望与应用拓展": these are the operations before and after
// the SSD that a deeper fusion takes into the SSD launch; the fused form is in ssd_tile16.h).
// Both are HBM-bound streams: each lane owns a piece of consecutive channels of a token row and
// consecutive lanes take consecutive pieces.  16-bit inputs only.
#include "ssd_device.h"

namespace ssd {

// conv: out[b,t,ch] = silu(bias[ch] + sum_k w[ch][k] * in[b, t-3+k, ch]), K = 4, where
// in[b, t<0, ch] = state[b][ch][t+3] (zeros without a state).  Each lane owns kConvCW channels
// (one 8-byte piece) over kConvRows consecutive tokens and slides a 3-row window down them.  The
// output goes to x [B,L,H*P], B [B,L,G*N] or C [B,L,G*N] by channel range (H*P and G*N are
// multiples of 8, so a piece never straddles two of them).  Measured on MI355X: 4 channels per
// lane (50 registers instead of 84, so more waves in flight) beat 8 by a fifth of the kernel's time,
// and 2 channels per lane were slower again.
constexpr int kConvRows = 16;
constexpr int kConvCW = 4;  // channels per lane

template <typename T, int CW> struct ConvVec { typedef typename TT<T>::v8 type; };
template <typename T> struct ConvVec<T, 4> { typedef typename TT<T>::v4 type; };

template <typename T, int CW> __global__ __launch_bounds__(256) void k_conv_silu(ConvArgs a) {
    typedef typename ConvVec<T, CW>::type v8;
    const int ch = a.hp + 2 * a.gn, npc = ch / CW, L = a.seqlen;
    const int nseg = (L + kConvRows - 1) / kConvRows;
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (item >= (int64_t)a.batch * nseg * npc) return;
    const int pc = (int)(item % npc);
    const int seg = (int)((item / npc) % nseg);
    const int b = (int)(item / ((int64_t)npc * nseg));
    const int c0 = pc * CW, t0 = seg * kConvRows;
    float w[4][CW], bias[CW], win[3][CW];
#pragma unroll
    for (int e = 0; e < CW; ++e) {
        const f32x4 wv = *(const f32x4*)(a.w + (size_t)(c0 + e) * 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k][e] = wv[k];
        bias[e] = a.bias ? a.bias[c0 + e] : 0.f;
    }
    const T* src = (const T*)a.xbc + (size_t)b * L * ch + c0;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int t = t0 - 3 + r;
        if (t >= 0) {
            const v8 v = *(const v8*)(src + (size_t)t * ch);
#pragma unroll
            for (int e = 0; e < CW; ++e) win[r][e] = (float)v[e];
        } else {
#pragma unroll
            for (int e = 0; e < CW; ++e)
                win[r][e] = a.state ? (float)((const T*)a.state)[((size_t)b * ch + c0 + e) * 3 + (t + 3)] : 0.f;
        }
    }
    T* dst;
    size_t rs;
    if (c0 < a.hp) {
        dst = (T*)a.x + (size_t)b * L * a.hp + c0;
        rs = a.hp;
    } else if (c0 < a.hp + a.gn) {
        dst = (T*)a.B + (size_t)b * L * a.gn + (c0 - a.hp);
        rs = a.gn;
    } else {
        dst = (T*)a.C + (size_t)b * L * a.gn + (c0 - a.hp - a.gn);
        rs = a.gn;
    }
    for (int i = 0; i < kConvRows; ++i) {
        const int t = t0 + i;
        if (t >= L) break;
        const v8 v = *(const v8*)(src + (size_t)t * ch);
        v8 o;
#pragma unroll
        for (int e = 0; e < CW; ++e) {
            const float cur = (float)v[e];
            const float s = bias[e] + w[0][e] * win[0][e] + w[1][e] * win[1][e] + w[2][e] * win[2][e] + w[3][e] * cur;
            o[e] = (T)silu_f(s);
            win[0][e] = win[1][e];
            win[1][e] = win[2][e];
            win[2][e] = cur;
        }
        *(v8*)(dst + (size_t)t * rs) = o;
    }
}

// gated norm: g = y * silu(z); out = g / sqrt(mean over the channel group of g^2 + eps) * w.
// One wave per (token, group): two passes over the group's pieces (the second re-reads y and z,
// from the L2), a wave-wide sum in between.
template <typename T> __global__ __launch_bounds__(256) void k_gated_norm(NormArgs a) {
    typedef typename TT<T>::v8 v8;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, group)
    if (row >= (int64_t)a.rows * a.groups) return;
    const int cg = a.hp / a.groups, np = cg / 8;
    const int64_t tok = row / a.groups;
    const int g = (int)(row % a.groups);
    const size_t base = (size_t)tok * a.hp + (size_t)g * cg;
    const T* yp = (const T*)a.y + base;
    const T* zp = (const T*)a.z + base;
    float ss = 0.f;
    for (int pc = lane; pc < np; pc += 64) {
        const v8 yv = *(const v8*)(yp + pc * 8), zv = *(const v8*)(zp + pc * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float gv = (float)yv[e] * silu_f((float)zv[e]);
            ss += gv * gv;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float rs = __builtin_amdgcn_rsqf(ss / (float)cg + a.eps);
    T* op = (T*)a.out + base;
    for (int pc = lane; pc < np; pc += 64) {
        const v8 yv = *(const v8*)(yp + pc * 8), zv = *(const v8*)(zp + pc * 8);
        const f32x4 w0 = *(const f32x4*)(a.w + g * cg + pc * 8), w1 = *(const f32x4*)(a.w + g * cg + pc * 8 + 4);
        v8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float gv = (float)yv[e] * silu_f((float)zv[e]);
            o[e] = (T)(gv * rs * (e < 4 ? w0[e] : w1[e - 4]));
        }
        *(v8*)(op + pc * 8) = o;
    }
}

// The same in one pass when a wave's share of the group fits in registers (at most MAXP pieces
// per lane): y silu(z) of every piece is kept in fp32 while the wave sums its squares, so y and
// z are read once.  The per-element values and the order of the sum are those of k_gated_norm,
// so the results are bit-identical.
template <typename T, int MAXP> __global__ __launch_bounds__(256) void k_gated_norm1(NormArgs a) {
    typedef typename TT<T>::v8 v8;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, group)
    if (row >= (int64_t)a.rows * a.groups) return;
    const int cg = a.hp / a.groups, np = cg / 8;
    const int64_t tok = row / a.groups;
    const int g = (int)(row % a.groups);
    const size_t base = (size_t)tok * a.hp + (size_t)g * cg;
    const T* yp = (const T*)a.y + base;
    const T* zp = (const T*)a.z + base;
    float gv[MAXP][8];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
        const int pc = lane + 64 * k;
        if (pc < np) {
            const v8 yv = *(const v8*)(yp + pc * 8), zv = *(const v8*)(zp + pc * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gv[k][e] = (float)yv[e] * silu_f((float)zv[e]);
                ss += gv[k][e] * gv[k][e];
            }
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float rs = __builtin_amdgcn_rsqf(ss / (float)cg + a.eps);
    T* op = (T*)a.out + base;
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
        const int pc = lane + 64 * k;
        if (pc < np) {
            const f32x4 w0 = *(const f32x4*)(a.w + g * cg + pc * 8), w1 = *(const f32x4*)(a.w + g * cg + pc * 8 + 4);
            v8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (T)(gv[k][e] * rs * (e < 4 ? w0[e] : w1[e - 4]));
            *(v8*)(op + pc * 8) = o;
        }
    }
}

template <typename T> hipError_t launch_conv_t(ConvArgs& a, hipStream_t st) {
    const int npc = (a.hp + 2 * a.gn) / kConvCW;
    const int64_t items = (int64_t)a.batch * ((a.seqlen + kConvRows - 1) / kConvRows) * npc;
    void* args[] = {&a};
    return hipLaunchKernel((const void*)&k_conv_silu<T, kConvCW>, dim3((unsigned)((items + 255) / 256)), dim3(256),
                           args, 0, st);
}

template <typename T> hipError_t launch_norm_t(NormArgs& a, hipStream_t st) {
    const int64_t waves = (int64_t)a.rows * a.groups;
    const int ppl = (a.hp / a.groups / 8 + 63) / 64;  // pieces per lane
    const void* fn = ppl <= 4 ? (const void*)&k_gated_norm1<T, 4>
                   : ppl <= 8 ? (const void*)&k_gated_norm1<T, 8>
                   : ppl <= 12 ? (const void*)&k_gated_norm1<T, 12> : (const void*)&k_gated_norm<T>;
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)((waves + 3) / 4)), dim3(256), args, 0, st);
}

hipError_t launch_conv_silu(ConvArgs& a, int in_dtype, hipStream_t st) {
    switch (in_dtype) {
    case DT_F16: return launch_conv_t<_Float16>(a, st);
    case DT_BF16: return launch_conv_t<__bf16>(a, st);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_gated_norm(NormArgs& a, int in_dtype, hipStream_t st) {
    switch (in_dtype) {
    case DT_F16: return launch_norm_t<_Float16>(a, st);
    case DT_BF16: return launch_norm_t<__bf16>(a, st);
    default: return hipErrorNotSupported;
    }
}

}  // namespace ssd
