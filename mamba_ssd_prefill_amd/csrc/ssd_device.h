// ssd_device.h -- gfx950 device code for the Mamba-2 SSD chunked prefill.
//
// Page keys used in comments:
//   [KF]  "Mamba-2炸裂升级！大模型推理飙升20%，效率翻2.5倍！" (repost of "Accelerating
//         Mamba2 with Kernel Fusion"); sections "Mamba-2核心操作与融合的必要性" (the five
//         SSD steps), "高效内核融合技术揭秘" (fused schedule), "性能瓶颈的深入分析"
//         (boundary split-out, decay on x, chunk size).
//   [HW]  "Mamba 硬件感知算法", sections "块分解与状态传递" (chunk decomposition) and
//         "Mamba-2 Segsum 稳定化" (decay kept in log space).
//   [XLA] "Mamba-2状态空间模型的编译器优化与实现", section 1.1 (the recurrence) and 2.2
//         (decay exponent kept in fp32).
//
// Tensor layouts (row-major): x, y [B][L][H][P]; dt [B][L][H]; B, C [B][L][G][N];
// states [B][K][H][P][N].  Workspace intermediates are described in mamba_ssd.h.
//
// MFMA conventions (16x16 output tiles, one 64-lane wave):
//   A operand: lane l holds row (l & 15), KPL consecutive k starting at KPL * (l >> 4);
//   B operand: lane l holds column (l & 15), the same k slots;
//   accumulator: lane l holds rows 4 * (l >> 4) + r (r = 0..3) of column (l & 15).
// Only the A/B symmetry of the k slots matters for a contraction, which lets the
// state held in accumulator layout feed the C . S^T product directly (see y_off).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_launch.h"

namespace ssd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// ---- element-type traits -------------------------------------------------------------
template <typename T> struct TT;
template <> struct TT<__bf16> {
    static constexpr int KPL = 8;  // k values per lane in one MFMA
    typedef bf16x8 frag;
    typedef bf16x8 v8;  // 16 bytes
    typedef bf16x4 v4;
    typedef bf16x2 v2;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct TT<_Float16> {
    static constexpr int KPL = 8;
    typedef f16x8 frag;
    typedef f16x8 v8;
    typedef f16x4 v4;
    typedef f16x2 v2;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct TT<float> {
    static constexpr int KPL = 1;
    typedef float frag;
    typedef f32x4 v8;  // 16 bytes
    typedef f32x4 v4;
    typedef f32x2 v2;
    __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename V> __device__ inline V vzero() {
    V v;
    __builtin_memset(&v, 0, sizeof(V));
    return v;
}

// ---- per-(T, P, N) geometry of a chunk tile --------------------------------------------
// A chunk tile is (chunk c, batch b, group g, a run of HPT heads of g).  Its four waves
// split as HPT heads x WPH p-slices of PW columns each.  Tokens are handled in windows
// of W = 64 (chunk sizes are multiples of 64).
template <typename T, int P, int N> struct Geo {
    static constexpr int W = 64;
    static constexpr int PW = P < 32 ? P : 32;
    static constexpr int WPH = P / PW;
    static constexpr int HPT = 4 / WPH;
    static constexpr int MBP = PW / 16;
    static constexpr int NB = N / 16;
    static constexpr int WB = W / 16;
    static constexpr int KPL = TT<T>::KPL;
    static constexpr int KI = 4 * KPL;
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr int PADE = 16 / (int)sizeof(T);  // 16 bytes of row padding
    static constexpr int LDW = W + PADE;
    static constexpr int LDN = N + PADE;
    static constexpr int QMAX = 256;
    static constexpr int SZ_BT = N * LDW * (int)sizeof(T);
    static constexpr int SZ_XW = HPT * P * LDW * (int)sizeof(T);
    static constexpr int SZ_C = W * LDN * (int)sizeof(T);
    static constexpr int SZ_L = HPT * W * LDW * (int)sizeof(T);
    static constexpr int SZ_XT = HPT * P * LDW * (int)sizeof(T);
    static constexpr int SZ_PHASE_S = SZ_BT + SZ_XW;
    static constexpr int SZ_PHASE_Y = SZ_C + SZ_L + SZ_XT;
    static constexpr int SZ_MAIN = SZ_PHASE_S > SZ_PHASE_Y ? SZ_PHASE_S : SZ_PHASE_Y;
    static constexpr int SZ_VEC = (3 * HPT + 1) * QMAX * 4;  // dt, acs, chunk-state weights; seg
    static constexpr int SMEM = SZ_MAIN + SZ_VEC;
    static_assert(P % 16 == 0 && N % 16 == 0, "P and N must be multiples of 16");
    static_assert(KPL == 1 || N % 32 == 0, "16-bit inputs need N % 32 == 0");
    static_assert(P <= 128, "P <= 128");
};

// ---- scalar helpers ------------------------------------------------------------------
// threadIdx.x through an opaque move.  Tile code that the fused kernel runs inside its work
// loop derives its lane offsets from this, so the compiler computes them where they are used
// on each trip instead of hoisting them out of the loop and keeping them all live.
__device__ inline int tid_here() {
    int t;
    asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
    return t;
}


__device__ inline float softplus_f(float z) {
    // log(1 + e^z) without overflow
    return z > 0.f ? z + log1pf(__expf(-z)) : log1pf(__expf(z));
}

template <typename T> __device__ inline float f32of(T v) { return (float)v; }

template <typename T> __device__ inline typename TT<T>::v4 cvt4(f32x4 v) {
    typename TT<T>::v4 o;
    o[0] = (T)v[0];
    o[1] = (T)v[1];
    o[2] = (T)v[2];
    o[3] = (T)v[3];
    return o;
}

template <typename T> __device__ inline typename TT<T>::frag load_frag(const T* p) {
    if constexpr (TT<T>::KPL == 8)
        return *(const typename TT<T>::frag*)p;
    else
        return *p;
}

// Buffer resource for [base, base + bytes); every caller passes wave-uniform values, which are
// made scalar explicitly so the descriptor lives in SGPRs (a descriptor the compiler cannot
// prove uniform is re-built per lane in a loop around every access).  Reads past `bytes`
// return zeros.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* p = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// ---- data shared between workgroups of one launch ------------------------------------------
// The fused kernel keeps every producer -> consumer hand-off (dt/acs, CB, the inter-chunk
// states and the flags that order them) inside one XCD: a chain's chunk tiles and the
// cumsum / bmm tiles they read belong to one work partition, served only by workgroups
// running on one XCD (see fused_loop).  On gfx950 (measured on MI355X):
//   * plain stores go through the CU's L1 into the XCD's L2, which is write-back: another
//     XCD does not see them until the kernel ends, a workgroup on the same XCD does;
//   * loads with sc1 set miss the CU's L1 and are served by the L2 (about 200 cycles when
//     the line is there); sc0 alone, and plain loads, may return a stale L1 copy, and
//     buffer_inv sc0 does not prevent that outside thread-group-split dispatches;
// so a producer stores plainly, waits for its stores (s_waitcnt vmcnt(0)) and raises a flag;
// the consumer polls the flag and reads the data with sc1 loads.  No cache-wide fence is
// needed: an agent-scope acquire / release would invalidate / write back the whole L2.
constexpr int AUX_L2 = 16;  // sc1

template <int AUX> __device__ inline float bload_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, AUX));
}
template <int AUX> __device__ inline f32x4 bload_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, AUX));
}

// 4 consecutive state elements in the state dtype, widened to / rounded from fp32.
__device__ inline f32x4 load_state4(const void* base, int dtype, size_t off) {
    if (dtype == DT_F32) return *((const f32x4*)((const float*)base + off));
    const uint64_t bits = *(const uint64_t*)((const uint16_t*)base + off);
    if (dtype == DT_F16) {
        const f16x4 v = __builtin_bit_cast(f16x4, bits);
        return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
    const bf16x4 v = __builtin_bit_cast(bf16x4, bits);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

__device__ inline void store_state4(void* base, int dtype, size_t off, f32x4 v) {
    if (dtype == DT_F32) {
        *(f32x4*)((float*)base + off) = v;
    } else if (dtype == DT_F16) {
        *(f16x4*)((uint16_t*)base + off) = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    } else {
        *(bf16x4*)((uint16_t*)base + off) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    }
}

// ---- cross-workgroup waits -------------------------------------------------------------
// Poll a flag word (sc1 loads, from the L2) until it reaches `target`.  Bounded: after spin_limit polls (or
// once any wait has given up) it raises the abort word and the status word -- device-scope
// accesses, since every partition must see them -- and returns false, so every workgroup
// still runs to completion.  All lanes of the calling wave poll the same address.
// Waiters further back sleep longer between polls (s_sleep n is about 64 n cycles): a chain's
// counter is polled by every waiting tile of the chain, and a tight loop from all of them
// would saturate its L2 channel -- slowing the very stores it waits for.
// Every 32nd poll of a wait, and every poll past spin_limit: false once another wait gave up or
// this one has polled more than spin_limit times (then it raises the abort and status words).
__device__ inline bool spin_ok(uint32_t spins, const SsdArgs& a) {
    if ((spins & 31u) != 0u && spins <= a.spin_limit) return true;
    if (__hip_atomic_load(a.abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return false;
    if (spins > a.spin_limit) {
        __hip_atomic_store(a.abort_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.status, 7u /* SSD_ERR_SYNC_TIMEOUT */, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    return true;
}

__device__ inline bool wait_flag(const uint32_t* f, const SsdArgs& a, uint32_t target = 1u) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(f, 4);
    uint32_t spins = 0;
    bool ok = true;
    uint32_t v;
    while ((v = __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, AUX_L2)) < target) {
        const uint32_t behind = target - v;  // hand-offs still to come before this one
        if (behind > 3u)
            __builtin_amdgcn_s_sleep(127);
        else if (behind > 1u)
            __builtin_amdgcn_s_sleep(24);
        if (!spin_ok(++spins, a)) {
            ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    // keeps the compiler from hoisting the reads of published data above the poll
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return ok;
}

// wait_flag over the first n (<= 64) words at f: returns once every one is >= target.
__device__ inline bool wait_words(const uint32_t* f, int n, const SsdArgs& a, uint32_t target) {
    const uint32_t lane = (uint32_t)tid_here() & 63u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(f, (uint32_t)n * 4);
    uint32_t spins = 0;
    bool ok = true;
    for (;;) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, lane * 4, 0, AUX_L2);
        const unsigned long long low = __ballot(lane < (uint32_t)n && v < target);
        if (low == 0ull) break;
        const uint32_t behind = target - __builtin_amdgcn_readlane(v, __builtin_ctzll(low));
        if (behind > 3u)
            __builtin_amdgcn_s_sleep(127);
        else if (behind > 1u)
            __builtin_amdgcn_s_sleep(24);
        if (!spin_ok(++spins, a)) {
            ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return ok;
}

// One wave: wait until base[o0] >= 1 and base[o1] >= 1 (lanes 0 and 1 poll one word each).
__device__ inline bool wait_pair(const uint32_t* base, uint32_t o0, uint32_t o1, const SsdArgs& a) {
    const uint32_t lane = (uint32_t)tid_here() & 63u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, ((o0 > o1 ? o0 : o1) + 1) * 4);
    const uint32_t off = (lane == 1 ? o1 : o0) * 4;
    uint32_t spins = 0;
    bool ok = true;
    for (;;) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX_L2);
        if (__ballot(lane < 2 && v < 1u) == 0ull) break;
        if (!spin_ok(++spins, a)) {
            ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return ok;
}

// A row of per-slot words (at most 32, one 128-byte line), one slot per item modulo `slots`:
// the number of consecutive items base, base + 1, ... (at most `slots`) whose slot word w
// has w + bias >= item + 1.  One sc1 load per lane; the result is wave-uniform.
__device__ inline int ready_run(const uint32_t* row, int slots, uint32_t base, uint32_t bias) {
    const uint32_t lane = (uint32_t)tid_here() & 63u;
    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(row, (uint32_t)slots * 4), lane * 4, 0, AUX_L2);
    const uint32_t s0 = base % (uint32_t)slots;
    const uint32_t k = (lane + (uint32_t)slots - s0) % (uint32_t)slots;  // item base + k lives in slot `lane`
    const unsigned long long bad = __ballot(lane < (uint32_t)slots && v + bias < base + k + 1u);
    const unsigned long long all = (1ull << slots) - 1ull;
    const unsigned long long rot = ((bad >> s0) | (bad << ((uint32_t)slots - s0))) & all;  // bit k: item base + k
    return rot ? __builtin_ctzll(rot) : slots;
}

// Polls ready_run until it is positive; bounded like wait_flag (0 when the wait gave up).
__device__ inline int wait_run(const uint32_t* row, int slots, uint32_t base, uint32_t bias, const SsdArgs& a) {
    uint32_t spins = 0;
    for (;;) {
        const int n = ready_run(row, slots, base, bias);
        if (n > 0) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            return n;
        }
        if (!spin_ok(++spins, a)) return 0;
        __builtin_amdgcn_s_sleep(1);
    }
}

// s_waitcnt vmcnt(0): every global load and store this wave issued has completed.
__device__ inline void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(n): at most the n most recent global loads / stores of this wave are still
// pending (vector memory operations complete in issue order; vmcnt is bits [3:0] and [15:14]).
template <int n> __device__ inline void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS accesses have completed
// (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() (whose workgroup fence waits for
// every outstanding global access too) it leaves global loads in flight, so a read issued
// early keeps overlapping whatever follows.  Also a compiler barrier for memory accesses.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ inline void raise_flag(uint32_t* f, uint32_t v = 1u) {
    __builtin_amdgcn_raw_buffer_store_b32(v, make_rsrc(f, 4), 0, 0, 0);
}

// Every lane: its stores have reached the L2, then set *f = v.
__device__ inline void publish_flag_wave(uint32_t* f, uint32_t v = 1u) {
    wait_vm_all();
    raise_flag(f, v);
}

// Per-chain progress counter of the fused form: one word per (b, h, p-slice) chain, alone in
// its 128-byte line, so the line stays resident in the L2 (a flag word that shares a line
// with cold data, or a first store that allocates a partial line, makes the next sc1 read
// go to memory).  Value v: the states entering chunks 0 .. v-1 are published.
__device__ inline uint32_t* chain_counter(const SsdArgs& a, int b, int h, int ph, int WPH) {
    return a.flags + (((size_t)b * a.nheads + h) * WPH + ph) * kChainStride;
}

// Whole workgroup: every wave's stores have reached the L2, then thread 0 sets *f.
__device__ inline void publish_flag_block(uint32_t* f) {
    wait_vm_all();
    __syncthreads();
    if (threadIdx.x == 0) raise_flag(f);
}

// ---- the fused form's inter-chunk state ring -----------------------------------------------
// Slot layout: for every (b, h, p-slice ph, slot) the owning wave's accumulator tiles follow
// each other, lane after lane: element e of tile t held by lane l sits at
// ring_chain(b, slot, h, ph) + (t * 64 + l) * 4 + e, where tile t = nb * MBP + pb covers
// S[p = ph*PW + pb*16 + (l & 15)][n = nb*16 + 4*(l >> 4) + e].  Each lane therefore moves one
// contiguous 16-byte (fp32) or 8-byte (16-bit) piece and a wave moves 1 KB / 512 B at once.
// The boundary copies convert between this layout and the callers' [P][N] layout.
__device__ inline size_t ring_chain(int b, int slot, int h, int ph, int K, int H, int WPH, int tiles) {
    return ((((size_t)b * H + h) * WPH + ph) * K + slot) * (size_t)tiles * 256;
}

// Load (sc1: from the XCD's L2) / plain store of one lane's 4 ring elements at element offset
// `off` of the chain whose descriptor is `r` (ring_rsrc).
__device__ inline __amdgpu_buffer_rsrc_t ring_rsrc(const void* states, int dtype, size_t chain, int tiles) {
    const int es = dtype == DT_F32 ? 4 : 2;
    return make_rsrc((const char*)states + chain * es, tiles * 256 * es);
}

__device__ inline f32x4 ring_load(__amdgpu_buffer_rsrc_t r, int dtype, uint32_t off) {
    if (dtype == DT_F32) return bload_f32x4<AUX_L2>(r, off * 4);
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off * 2, 0, AUX_L2);
    if (dtype == DT_F16) {
        const f16x4 v = __builtin_bit_cast(f16x4, w);
        return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
    const bf16x4 v = __builtin_bit_cast(bf16x4, w);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

__device__ inline void ring_store(__amdgpu_buffer_rsrc_t r, int dtype, uint32_t off, f32x4 v) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if (dtype == DT_F32) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off * 4, 0, 0);
    } else if (dtype == DT_F16) {
        const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, off * 2, 0, 0);
    } else {
        const bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, off * 2, 0, 0);
    }
}

// ---- the relay form of the fused state passing ---------------------------------------------
// With few chains per XCD the chunk-to-chunk hop inside the chunk tiles (each tile reads S_c,
// writes S_{c+1} and releases the next tile) bounds the whole launch: its latency is paid once
// per chunk, in series, and one wave issues a vector memory instruction only every few tens of
// nanoseconds, so moving a wave's 16 KB of state costs microseconds.  The relay form gives every
// chain (b, h, p-slice) a dedicated state-passing item whose relay waves each keep a share of S
// (whole accumulator tiles) in fp32 registers and stream the chunk states through:
//   chunk tile c:  s_c -> chunk-state ring slot c % agg_slots (fp32; fp16 with fp16 state
//                  storage), slot word = c + 1; wait
//                  until every relay wave's counter >= c + 1, read S_c (operand type) from
//                  operand slot c % op_slots, read word = c + 1
//   relay wave:    for c = 0, 1, ...: S_{c+1} = exp(acs_c[Q-1]) S_c + s_c (its tiles) -> operand
//                  slot (c + 1) % op_slots, its counter = c + 2 once stored; first S_0 (from
//                  state ring slot 0) -> operand slot 0, counter = 1; at the end S_nc in the
//                  state dtype -> state ring slot 1
// The tiles read S_c only as an MFMA operand, so the relay hands it over already rounded to
// the operand type (half the bytes and instructions of fp32).  A chunk tile overwrites its
// chunk-state slot only after every relay wave has used the previous occupant (counters >=
// c - agg_slots + 2); a relay wave overwrites an operand slot only after the tile that read the
// previous occupant said so (read word).  A relay wave loads s_{c+1} while s_c is being folded
// in and publishes S_c one chunk later, once its stores are known complete.  Both rings keep
// each lane's 16-byte pieces contiguous (see ring_chain): a chunk-state slot holds the NT
// accumulator tiles as fp32, an operand slot holds them in units of 16 / (4 sizeof(T)) tiles.
template <typename T> constexpr int tiles_per_unit() { return sizeof(T) == 2 ? 2 : 1; }

// Relay waves of a chain whose chunk-tile wave holds NT accumulator tiles, at most RWM (the
// launch's choice, 2 or 4): each relay wave takes the same number of whole operand units.
template <typename T, int NT, int RWM> constexpr int relay_waves() {
    return NT / tiles_per_unit<T>() < RWM ? NT / tiles_per_unit<T>() : RWM;
}
template <typename T, int NT> __device__ inline int relay_waves_of(const SsdArgs& a) {
    return a.relay == 4 ? relay_waves<T, NT, 4>() : relay_waves<T, NT, 2>();
}

__device__ inline size_t chain_index(const SsdArgs& a, int b, int h, int ph, int WPH) {
    return ((size_t)b * a.nheads + h) * WPH + ph;
}

// The chunk-state ring slot of chain (b, h, ph): NT accumulator tiles of 64 lanes x 4 floats,
// lane after lane as in ring_chain.  a.agg16: 4 fp16 instead, tiles 2u and 2u + 1 of a lane
// side by side in its 16-byte unit u (unit u of lane l at byte (u * 64 + l) * 16).
// c modulo the ring size, which is one of two constants (a division by an unknown divisor
// would lengthen every step of the relay's serial chain)
__device__ inline int agg_slot(const SsdArgs& a, int c) {
    return a.agg_slots == kAggSlotsLong ? c % kAggSlotsLong : c % kAggSlots;
}

template <int NT> __device__ inline __amdgpu_buffer_rsrc_t agg_rsrc(const SsdArgs& a, int b, int h, int ph, int WPH,
                                                                     int slot) {
    const size_t chain = chain_index(a, b, h, ph, WPH) * a.agg_slots + slot;
    const int es = a.agg16 ? 2 : 4;
    return make_rsrc((const char*)a.s + chain * NT * 256 * es, NT * 256 * es);
}

// The operand ring slot of chain (b, h, ph): NT tiles of 64 lanes x 4 elements of T.
template <typename T, int NT>
__device__ inline __amdgpu_buffer_rsrc_t opnd_rsrc(const SsdArgs& a, int b, int h, int ph, int WPH, int slot) {
    const size_t chain = chain_index(a, b, h, ph, WPH) * a.op_slots + slot;
    return make_rsrc((const T*)a.opnd + chain * NT * 256, NT * 256 * sizeof(T));
}

// 16 bytes of operand ring: tiles u * TPU .. u * TPU + TPU - 1 of one lane, rounded to T.
template <typename T> __device__ inline u32x4 pack_unit(const f32x4* v) {
    if constexpr (sizeof(T) == 2) {
        typedef typename TT<T>::v4 v4;
        const v4 lo = cvt4<T>(v[0]), hi = cvt4<T>(v[1]);
        return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
        return __builtin_bit_cast(u32x4, v[0]);
    }
}

// Relay wave w of chain (b, h, ph): the state passing of tiles [w * TPW, (w + 1) * TPW) of the
// chain's NT accumulator tiles, over every chunk.  VL: packed variable-length input.  With
// a.agg16 the chunk-state ring holds fp16: the wave's TPW tiles arrive in TPW / 2 16-byte loads,
// and the other TPW / 2 loads go to an empty buffer range (no memory access, zeros), so the
// number of memory operations per chunk -- which the waits below count -- stays the same.  (A
// run-time choice rather than another instantiation: four relay instantiations in the fused
// kernel pushed its registers into spills.)
template <typename T, int NT, int RWM, int VL>
__device__ void relay_chain(const SsdArgs& a, int b, int h, int ph, int WPH, int w) {
    constexpr int TPU = tiles_per_unit<T>(), TPW = NT / relay_waves<T, NT, RWM>();
    static_assert(TPW % TPU == 0, "a relay wave holds whole operand units");
    constexpr int NAL = TPW;  // chunk-state loads per chunk (one per tile)
    const uint32_t lane = (uint32_t)tid_here() & 63u;
    const int H = a.nheads, nc = a.nchunks, Q = a.chunk, K = a.slots, KO = a.op_slots, sdt = a.state_dtype;
    uint32_t* cnt = chain_counter(a, b, h, ph, WPH);
    uint32_t* my_cnt = cnt + w;
    const uint32_t* agg_words = cnt + kChainAggWords;
    const uint32_t* read_words = cnt + kChainReadWords;
    const uint32_t t0 = (uint32_t)(w * TPW);
    f32x4 S[TPW];
    typedef u32x4 aggv;  // one lane's 4 fp32 elements of a tile, or (fp16) of two tiles
    aggv B0[NAL], B1[NAL];
    const bool a16 = a.agg16;
    static_assert(TPW % 2 == 0 || sizeof(T) == 4, "16-bit tiles come in pairs");
    float d0 = 0.f, d1 = 0.f;
    uint32_t g0 = 0u, g1 = 0u;
    {
        const __amdgpu_buffer_rsrc_t r = ring_rsrc(a.states, sdt, ring_chain(b, 0, h, ph, K, H, WPH, NT), NT);
#pragma unroll
        for (int t = 0; t < TPW; ++t) S[t] = a.has_h0 ? ring_load(r, sdt, ((t0 + t) * 64 + lane) * 4) : vzero<f32x4>();
        // S_0 into operand slot 0, then published (the counters start at 0 in this form)
        const __amdgpu_buffer_rsrc_t ro = opnd_rsrc<T, NT>(a, b, h, ph, WPH, 0);
#pragma unroll
        for (int u = 0; u < TPW / TPU; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(pack_unit<T>(&S[u * TPU]), ro, ((t0 / TPU + u) * 64 + lane) * 16, 0, 0);
        publish_flag_wave(my_cnt, 1u);
    }
    int agg_hi = 0;  // chunk states 0 .. agg_hi - 1 are known to be in their slots
    int wr_hi = 0;   // states 0 .. wr_hi - 1 are known to be free to write
    // L(c): TPW loads of s_c, one of acs_c[Q-1] and (packed input) one of seg_c[Q-1], nonzero
    // when a sequence starts inside chunk c, which then passes no state on; into buf / d / sg
    auto issue_load = [&](int c, aggv (&buf)[NAL], float& d, uint32_t& sg) {
        const __amdgpu_buffer_rsrc_t r = agg_rsrc<NT>(a, b, h, ph, WPH, agg_slot(a, c));
        const __amdgpu_buffer_rsrc_t rnone = make_rsrc(a.s, 0u);
#pragma unroll
        for (int t = 0; t < NAL; ++t) {
            const bool real = !a16 || 2 * t < TPW;
            const uint32_t unit = a16 ? t0 / 2 + t : t0 + t;
            buf[t] = __builtin_amdgcn_raw_buffer_load_b128(real ? r : rnone, (unit * 64 + lane) * 16, 0, AUX_L2);
        }
        d = bload_f32<AUX_L2>(make_rsrc(a.acs + (((size_t)b * nc + c) * H + h) * Q, (uint32_t)Q * 4),
                              (uint32_t)(Q - 1) * 4);
        if constexpr (VL != 0)
            sg = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.seg + ((size_t)b * nc + c) * Q, (uint32_t)Q * 4),
                                                      (uint32_t)(Q - 1) * 4, 0, AUX_L2);
        else
            sg = 0u;
    };
    // Step c: issue L(c + 1) if s_{c+1} is known to be ready, wait for L(c), publish S_{c-1},
    // else wait for s_{c+1} and issue L(c + 1) now; fold s_c in; store S_{c+1} (St(c + 1),
    // TPW / TPU stores).  Issue order: ... L(c), St(c), L(c + 1), St(c + 1) ...: once at most
    // |St(c)| + |L(c + 1)| operations are pending (|St(c)| alone if L(c + 1) is not issued yet),
    // L(c) and everything before it (St(c - 1) too) are complete.  Any extra operation in
    // between (a poll, a flag) only makes the count wait for more.
    constexpr int NST = TPW / TPU, NLD = NAL + (VL != 0 ? 2 : 1);
    auto step = [&](int c, aggv (&cur)[NAL], float dcur, uint32_t gcur, aggv (&nxt)[NAL], float& dnxt,
                    uint32_t& gnxt) -> bool {
        const bool has_next = c + 1 < nc;
        const bool early = has_next && c + 1 < agg_hi;
        if (early) issue_load(c + 1, nxt, dnxt, gnxt);
        asm volatile("" ::: "memory");
        if (early) {
            if (c >= 1)
                wait_vm<NST + NLD>();
            else
                wait_vm<NLD>();
        } else {
            if (c >= 1)
                wait_vm<NST>();
            else
                wait_vm<0>();
        }
        asm volatile("" ::: "memory");
        if (c >= 2) raise_flag(my_cnt, (uint32_t)c);  // states entering chunks 0 .. c-1 are stored
        if (has_next && !early) {
            // about to wait for s_{c+1} anyway: let St(c) complete and publish S_c now, so
            // chunk tile c does not wait for chunk tile c + 1
            if (c >= 1) {
                wait_vm<0>();
                raise_flag(my_cnt, (uint32_t)c + 1);
            }
            const int n = wait_run(agg_words, a.agg_slots, (uint32_t)c + 1, 0u, a);
            if (n == 0) return false;
            agg_hi = c + 1 + n;
            asm volatile("" ::: "memory");
            issue_load(c + 1, nxt, dnxt, gnxt);
            asm volatile("" ::: "memory");
        }
        const float dec = gcur ? 0.f : __expf(dcur);
        if (a16) {
#pragma unroll
            for (int u = 0; u < TPW / 2; ++u) {
                const f16x8 hv = __builtin_bit_cast(f16x8, cur[u]);
                S[2 * u] = dec * S[2 * u] + f32x4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]};
                S[2 * u + 1] = dec * S[2 * u + 1] + f32x4{(float)hv[4], (float)hv[5], (float)hv[6], (float)hv[7]};
            }
        } else {
#pragma unroll
            for (int t = 0; t < TPW; ++t) S[t] = dec * S[t] + __builtin_bit_cast(f32x4, cur[t]);
        }
        const int m = c + 1;  // the state written now
        if (m >= wr_hi) {
            // slot m % KO last held S_{m-KO}: its reader must be done (bias KO: always true for m < KO)
            const int n = wait_run(read_words, KO, (uint32_t)m, (uint32_t)KO, a);
            if (n == 0) return false;
            wr_hi = m + n;
        }
        asm volatile("" ::: "memory");
        const __amdgpu_buffer_rsrc_t r = opnd_rsrc<T, NT>(a, b, h, ph, WPH, m % KO);
#pragma unroll
        for (int u = 0; u < NST; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(pack_unit<T>(&S[u * TPU]), r,
                                                   ((t0 / TPU + u) * 64 + lane) * 16, 0, 0);
        asm volatile("" ::: "memory");
        return true;
    };
    bool ok = true;
    {
        const int n = wait_run(agg_words, a.agg_slots, 0u, 0u, a);
        ok = n > 0;
        agg_hi = n;
    }
    if (ok) issue_load(0, B0, d0, g0);
    for (int c = 0; ok && c < nc; c += 2) {
        ok = step(c, B0, d0, g0, B1, d1, g1);
        if (ok && c + 1 < nc) ok = step(c + 1, B1, d1, g1, B0, d0, g0);
    }
    // the final state, in the state dtype, for the boundary copy
    const __amdgpu_buffer_rsrc_t rf = ring_rsrc(a.states, sdt, ring_chain(b, 1, h, ph, K, H, WPH, NT), NT);
#pragma unroll
    for (int t = 0; t < TPW; ++t) ring_store(rf, sdt, ((t0 + t) * 64 + lane) * 4, S[t]);
    wait_vm_all();
    if (ok) raise_flag(my_cnt, (uint32_t)nc + 1);
}

// Relay form, chunk tile side: hand this wave's chunk state s_c (accumulator tiles) to the
// chain's relay waves, then read S_c (operand type) into sv.  False when a wait gave up.
template <typename T, int NB, int MBP>
__device__ inline bool relay_handoff(const SsdArgs& a, int b, int c, int h, int ph, int WPH,
                                     const f32x4 (&acc)[NB][MBP], typename TT<T>::v4 (&sv)[NB][MBP]) {
    constexpr int NT = NB * MBP, TPU = tiles_per_unit<T>();
    const int RW = relay_waves_of<T, NT>(a);
    typedef typename TT<T>::v4 v4;
    const uint32_t lane = (uint32_t)tid_here() & 63u;
    uint32_t* cnt = chain_counter(a, b, h, ph, WPH);
    // the slot's previous chunk state (chunk c - agg_slots) has been folded in
    const int KA = a.agg_slots;
    bool ok = c < KA || wait_words(cnt, RW, a, (uint32_t)(c - KA) + 2u);
    const __amdgpu_buffer_rsrc_t ra = agg_rsrc<NT>(a, b, h, ph, WPH, agg_slot(a, c));
    if (a.agg16) {
        // tile t of this lane: 8 bytes at ((t / 2) * 64 + lane) * 16 + (t % 2) * 8
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) {
                const uint32_t t = (uint32_t)(nb * MBP + pb);
                const f32x4 v = acc[nb][pb];
                const f16x4 hv = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, hv), ra,
                                                      ((t >> 1) * 64 + lane) * 16 + (t & 1) * 8, 0, 0);
            }
    } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[nb][pb]), ra,
                                                       ((uint32_t)(nb * MBP + pb) * 64 + lane) * 16, 0, 0);
    }
    publish_flag_wave(cnt + kChainAggWords + agg_slot(a, c), (uint32_t)c + 1);
    ok = wait_words(cnt, RW, a, (uint32_t)c + 1) && ok;
    const int KO = a.op_slots;
    const __amdgpu_buffer_rsrc_t rin = opnd_rsrc<T, NT>(a, b, h, ph, WPH, c % KO);
    v4 unit[NT];
#pragma unroll
    for (int u = 0; u < NT / TPU; ++u) {
        const u32x4 w = __builtin_bit_cast(u32x4, bload_f32x4<AUX_L2>(rin, ((uint32_t)u * 64 + lane) * 16));
        if constexpr (TPU == 2) {
            typedef typename TT<T>::frag frag;
            const frag f = __builtin_bit_cast(frag, w);
            unit[2 * u] = __builtin_shufflevector(f, f, 0, 1, 2, 3);
            unit[2 * u + 1] = __builtin_shufflevector(f, f, 4, 5, 6, 7);
        } else {
            unit[u] = __builtin_bit_cast(v4, w);
        }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int pb = 0; pb < MBP; ++pb) sv[nb][pb] = unit[nb * MBP + pb];
    wait_vm_all();
    raise_flag(cnt + kChainReadWords + c % KO, (uint32_t)c + 1);
    return ok;
}

// ---- step 1: chunk_cumsum ([KF] item 4; [HW] segsum section: decay in log space) ------
// For one (b, c) and heads [h0, h1): dt = softplus(dt_raw + dt_bias) (0 past L) and the
// inclusive in-chunk running sum of dt * A, both fp32, into dtf / acs [B][nc][H][Q].  One
// wave per head; each lane owns Q/64 consecutive tokens, then a wave-wide exclusive scan of
// the lane totals.
// Packed variable-length input ([KF] "与vLLM的深度融合": sequences told apart by a per-token
// sequence index and masked, not offset): a token t > 0 whose seq_idx differs from token
// t - 1's starts a new sequence.  acs stays the plain in-chunk sum; wave 0 also writes
// seg[b][c][i] = the number of sequence starts among chunk tokens 0 .. i (tokens past L add
// none).  Two tokens i >= j of a chunk belong to one sequence exactly when seg[i] == seg[j]
// (sequences are contiguous), and the state entering the chunk reaches token i exactly when
// seg[i] == 0; every later step masks its decays with these tests, so nothing crosses a
// sequence start and the in-chunk sums lose no precision to the masking.
template <typename T> __device__ void cumsum_tile(const SsdArgs& a, int b, int c, int h0, int h1) {
    const int tid = tid_here(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Q = a.chunk, L = a.seqlen, H = a.nheads, nc = a.nchunks;
    const int V = Q >> 6;  // 1..4
    const T* dtr = (const T*)a.dt;
    for (int h = h0 + wave; h < h1; h += 4) {
        const float bias = a.dt_bias ? a.dt_bias[h] : 0.f;
        const float Ah = a.A[h];
        float d[4], run[4];
        float tot = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            d[k] = 0.f;
            if (k < V) {
                const int t = c * Q + lane * V + k;
                if (t < L) {
                    const float z = f32of(dtr[((size_t)b * L + t) * H + h]) + bias;
                    d[k] = a.softplus ? softplus_f(z) : z;
                }
                tot += d[k] * Ah;
            }
            run[k] = tot;
        }
        float incl = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        const float excl = incl - tot;
        const size_t base = (((size_t)b * nc + c) * H + h) * Q + (size_t)lane * V;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k < V) {
                a.dtf[base + k] = d[k];
                a.acs[base + k] = excl + run[k];
            }
    }
    if (a.seq_idx && wave == 0) {
        const int* sq = a.seq_idx + (size_t)b * L;
        int run[4], tot = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (k < V) {
                // with per-sequence states a row's first token starts a sequence as well
                const int t = c * Q + lane * V + k;
                tot += (t < L && (t > 0 ? sq[t] != sq[t - 1] : a.seqstates != 0)) ? 1 : 0;
            }
            run[k] = tot;
        }
        int incl = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        const size_t base = ((size_t)b * nc + c) * Q + (size_t)lane * V;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k < V) a.seg[base + k] = incl - tot + run[k];
    }
}

// The Q x Q block of CB number idx in a.cb (fp32, or with a.cb16 the 16-bit input type).
__device__ inline float* cb_at(const SsdArgs& a, size_t idx) {
    return (float*)((char*)a.cb + idx * (size_t)a.chunk * a.chunk * (a.cb16 ? 2 : 4));
}

// ---- per-sequence states of packed input ---------------------------------------------------
// The chunk's segments (the pieces of its sequences, [KF] "与vLLM的深度融合": one pseudo-chunk per
// sequence in a chunk) are numbered by seg: segment k holds the tokens with seg[i] == k.

// First token of the chunk with seg >= k (Q when none): wave-uniform, one LDS read per lane
// per 64 tokens (Q is a multiple of 64).
__device__ inline int seg_first(const int* sSeg, int Q, int k) {
    const int lane = tid_here() & 63;
    for (int w0 = 0; w0 < Q; w0 += 64) {
        const unsigned long long m = __ballot(sSeg[w0 + lane] >= k);
        if (m) return w0 + __builtin_ctzll(m);
    }
    return Q;
}

// Sequence number of token t of row b (wave-uniform).
__device__ inline int seq_at(const SsdArgs& a, int b, int t) {
    return __builtin_amdgcn_readfirstlane(a.seq_idx[(size_t)b * a.seqlen + t]);
}

// Element offset of state element (p, n) of head h of sequence q in a [nseq][H][P][N] array.
__device__ inline size_t seq_state_off(const SsdArgs& a, int q, int h, int p, int n, int P, int N) {
    return (((size_t)q * a.nheads + h) * P + p) * N + n;
}

// ---- step 2: bmm ([KF] item 7) ---------------------------------------------------------
// CB[i][j] = sum_n C_i[n] B_j[n] for one (b, c, g) into cbase[Q][Q], computed as CB^T blocks
// (rows j, columns i) so each lane stores 4 consecutive j of one row i.  Only blocks with
// i-block >= j-block are formed: the scan step reads j <= i only.  Fragments come straight
// from global memory (rows are n-contiguous).  With a.cb16 (the relaxed intermediates of
// "Mamba-2炸裂升级！…", section "精度与性能的平衡艺术") CB is rounded to the 16-bit input type.
template <typename T, int N> __device__ void bmm_tile(const SsdArgs& a, int b, int c, int g, float* cbase) {
    constexpr int KPL = TT<T>::KPL, KI = 4 * KPL;
    const int tid = tid_here(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, r16 = lane & 15;
    const int Q = a.chunk, L = a.seqlen, G = a.ngroups;
    const int QB = Q >> 4;
    const T* Bp = (const T*)a.B;
    const T* Cp = (const T*)a.C;
    typedef typename TT<T>::frag frag;
    for (int jb = wave; jb < QB; jb += 4) {
        const int tj = c * Q + jb * 16 + r16;
        frag af[N / KI];
#pragma unroll
        for (int ks = 0; ks < N / KI; ++ks)
            af[ks] = tj < L ? load_frag<T>(Bp + (((size_t)b * L + tj) * G + g) * N + ks * KI + q * KPL)
                            : vzero<frag>();
        for (int ib = jb; ib < QB; ++ib) {
            const int ti = c * Q + ib * 16 + r16;
            f32x4 acc = vzero<f32x4>();
#pragma unroll
            for (int ks = 0; ks < N / KI; ++ks) {
                const frag bf = ti < L ? load_frag<T>(Cp + (((size_t)b * L + ti) * G + g) * N + ks * KI + q * KPL)
                                       : vzero<frag>();
                acc = TT<T>::mma(af[ks], bf, acc);
            }
            const size_t o = (size_t)(ib * 16 + r16) * Q + jb * 16 + 4 * q;
            if constexpr (sizeof(T) == 2) {
                if (a.cb16) {
                    *(typename TT<T>::v4*)((T*)cbase + o) = cvt4<T>(acc);
                    continue;
                }
            }
            *(f32x4*)(cbase + o) = acc;
        }
    }
}

// ---- the convolution before the SSD, inside the fused launch -----------------------------
// silu(v) = v / (1 + e^-v) in fp32.
__device__ inline float silu_f(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

// Conv taps (width 4) and bias of channels ch0 .. ch0 + 7.
struct ConvTaps {
    float w[4][8], bias[8];
    __device__ inline void load(const float* conv_w, const float* conv_b, int ch0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const f32x4 wv = *(const f32x4*)(conv_w + (size_t)(ch0 + e) * 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k][e] = wv[k];
            bias[e] = conv_b ? conv_b[ch0 + e] : 0.f;
        }
    }
};

// The block form's convolution inputs, read once from the argument block (helpers take this
// rather than the argument block itself).
template <typename T> struct ConvSrc {
    const T* xbc;         // [B][L][ch]
    const T* state;       // [B][ch][3] or nullptr
    const float* w;       // [ch][4]
    const float* bias;    // [ch] or nullptr
    int ch, L;
    __device__ inline explicit ConvSrc(const SsdArgs& a)
        : xbc((const T*)a.xbc), state((const T*)a.conv_state), w(a.conv_w), bias(a.conv_b), ch(a.x_stride),
          L(a.seqlen) {}
    // raw input of channels ch0 .. ch0 + 7 of token t of batch row b, as fp32: the xBC row for
    // t >= 0, the conv state (the 3 inputs before token 0) or zeros for t < 0
    __device__ inline void raw(int b, int t, int ch0, float (&v)[8]) const {
        typedef typename TT<T>::v8 v8;
        if (t >= 0) {
            const v8 r = *(const v8*)(xbc + ((size_t)b * L + t) * ch + ch0);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (float)r[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = state ? (float)state[((size_t)b * ch + ch0 + e) * 3 + (t + 3)] : 0.f;
        }
    }
};

// Eight consecutive outputs of one 8-channel piece from its 11 inputs in[0..10] (tokens
// t0 - 3 .. t0 + 7): out[i] = silu(bias + sum_k w[k] in[i + k]).
template <typename T> __device__ inline void conv8(const ConvTaps& k, const float (&in)[11][8], typename TT<T>::v8 (&out)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            out[i][e] = (T)silu_f(k.bias[e] + k.w[0][e] * in[i][e] + k.w[1][e] * in[i + 1][e] + k.w[2][e] * in[i + 2][e] +
                                  k.w[3][e] * in[i + 3][e]);
}

// Block form, before the bmm tile of (b, c, g): B and C of the chunk's tokens from the raw xBC
// rows (channels H*P + g*N .. and H*P + G*N + g*N ..) through the convolution, into a.B / a.C
// ([B][L][G][N], the layout of the plain inputs) for the bmm tile and the chunk tiles that read
// them.  Items: (B or C, 8-channel piece, 8 tokens).
template <typename T, int N> __device__ __forceinline__ void conv_bc_tile(const SsdArgs& a, int b, int c, int g) {
    typedef typename TT<T>::v8 v8;
    const int Q = a.chunk, L = a.seqlen, Gn = a.ngroups, hp = a.xbc_hp;
    T* const Bw = (T*)a.B;
    T* const Cw = (T*)a.C;
    const ConvSrc<T> src(a);
    const int tok0 = c * Q;
    constexpr int NPC = N / 8;
    const int items = 2 * NPC * (Q / 8);
    for (int it = tid_here(); it < items; it += 256) {
        const int which = it / (NPC * (Q / 8));  // 0: B, 1: C
        const int rest = it - which * NPC * (Q / 8);
        const int seg = rest / NPC, pc = rest - seg * NPC;
        const int t0 = tok0 + seg * 8;
        if (t0 >= L) continue;
        const int ch0 = hp + which * Gn * N + g * N + pc * 8;
        ConvTaps k;
        k.load(src.w, src.bias, ch0);
        float in[11][8];
#pragma unroll
        for (int r = 0; r < 11; ++r) {
            const int t = t0 - 3 + r;
            if (t < L) src.raw(b, t, ch0, in[r]);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) in[r][e] = 0.f;
            }
        }
        v8 out[8];
        conv8<T>(k, in, out);
        T* dst = (which ? Cw : Bw) + (((size_t)b * L + t0) * Gn + g) * N + pc * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (t0 + i < L) *(v8*)(dst + (size_t)i * Gn * N) = out[i];
    }
}

// ---- LDS staging helpers ---------------------------------------------------------------
// Rows [t0, t0 + W) of a row-major [token][COLS] slice (row stride `rs` elements), stored
// transposed: dst[col][jj] with row length LDW, zeros for tokens >= L.  Two consecutive
// tokens per item so each LDS write packs a (jj, jj+1) pair.  When `scale` is given,
// row jj is multiplied by scale[jj] in fp32 before rounding.  nullptr src = zeros.
template <typename T, int COLS, int W, int LDW>
__device__ inline void stage_transposed(T* dst, const T* src, size_t rs, int t0, int L, const float* scale,
                                        int item0, int nthreads) {
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int NV = COLS / VEC;
    constexpr int CL = NV < 4 ? NV : 4;
    constexpr int ITEMS = (W / 2) * NV;
    typedef typename TT<T>::v8 v8;
    typedef typename TT<T>::v2 v2;
    for (int it = item0; it < ITEMS; it += nthreads) {
        const int cl = it % CL;
        const int jp = (it / CL) % (W / 2);
        const int ch = it / (CL * (W / 2));
        const int cv = ch * CL + cl;
        const int jj = 2 * jp;
        v8 v0 = vzero<v8>(), v1 = vzero<v8>();
        if (src) {
            if (t0 + jj < L) v0 = *(const v8*)(src + (size_t)(t0 + jj) * rs + cv * VEC);
            if (t0 + jj + 1 < L) v1 = *(const v8*)(src + (size_t)(t0 + jj + 1) * rs + cv * VEC);
            if (scale) {
                const float s0 = scale[jj], s1 = scale[jj + 1];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    v0[e] = (T)((float)v0[e] * s0);
                    v1[e] = (T)((float)v1[e] * s1);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            v2 pr;
            pr[0] = v0[e];
            pr[1] = v1[e];
            *(v2*)(dst + (cv * VEC + e) * LDW + jj) = pr;
        }
    }
}

// Rows [t0, t0 + W) of a [token][COLS] slice stored as-is: dst[row][col], row length LD.
template <typename T, int COLS, int W, int LD>
__device__ inline void stage_rows(T* dst, const T* src, size_t rs, int t0, int L) {
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int NV = COLS / VEC;
    typedef typename TT<T>::v8 v8;
    for (int it = threadIdx.x; it < W * NV; it += 256) {
        const int cv = it % NV, r = it / NV;
        v8 v = vzero<v8>();
        if (t0 + r < L) v = *(const v8*)(src + (size_t)(t0 + r) * rs + cv * VEC);
        *(v8*)(dst + r * LD + cv * VEC) = v;
    }
}

// ---- steps 3-5 on one chunk tile ---------------------------------------------------------
enum : int { MODE_STATE = 0, MODE_SCAN = 1, MODE_FUSED = 2 };

// MODE_STATE  chunk_state ([KF] item 5): s_c = sum_j x_j w_j (outer) B_j with
//             w_j = exp(acs[Q-1] - acs[j]) dt_j (decay applied to x, [KF] bottleneck
//             section) -> workspace s.
// MODE_SCAN   chunk_scan ([KF] item 8): y_i = exp(acs_i) C_i . S_c
//             + sum_{j<=i} CB[i][j] exp(acs_i - acs_j) dt_j x_j + D x_i, with S_c read
//             from the states slot of chunk c.
// MODE_FUSED  chunk_state, then the state_passing hop ([KF] item 6; fused schedule of
//             [KF] "高效内核融合技术揭秘"): wait for S_c, write S_{c+1} = exp(acs[Q-1]) S_c
//             + s_c to the next ring slot and release it, then chunk_scan with S_c.
// relay_live (MODE_FUSED of a relay-form launch): the partition's relay items run.  VL: packed
// variable-length input (a.seq_idx set), a separate instantiation.
template <typename T, int P, int N, int MODE, int VL>
__device__ void chunk_tile(const SsdArgs& a, int b, int c, int g, int tig, char* smem, const float* cbase,
                           bool relay_live = false) {
    typedef Geo<T, P, N> G_;
    constexpr int W = G_::W, PW = G_::PW, WPH = G_::WPH, HPT = G_::HPT, MBP = G_::MBP;
    constexpr int NB = G_::NB, WB = G_::WB, KPL = G_::KPL, KI = G_::KI, LDW = G_::LDW, LDN = G_::LDN;
    constexpr int QMAX = G_::QMAX;
    typedef typename TT<T>::frag frag;
    typedef typename TT<T>::v4 v4;

    constexpr int AUX = MODE == MODE_FUSED ? AUX_L2 : 0;  // data handed over inside one launch
    const int tid = tid_here(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, r16 = lane & 15;
    const int hs = wave / WPH, ph = wave % WPH;
    const int Q = a.chunk, L = a.seqlen, H = a.nheads, Gn = a.ngroups, nc = a.nchunks, hpg = a.hpg;
    const int head0 = g * hpg + tig * HPT;
    const int h = head0 + hs;
    const bool hvalid = (tig * HPT + hs) < hpg;
    const int tok0 = c * Q;
    const T* xg = (const T*)a.x;
    const T* Bg = (const T*)a.B;
    const T* Cg = (const T*)a.C;

    float* sDt = (float*)(smem + G_::SZ_MAIN);  // [HPT][QMAX]
    float* sAcs = sDt + HPT * QMAX;             // [HPT][QMAX]
    float* sW = sAcs + HPT * QMAX;              // [HPT][QMAX] chunk-state weights
    int* sSeg = (int*)(sW + HPT * QMAX);        // [QMAX] packed input: sequence starts up to token i
    constexpr bool varlen = VL != 0;

    {
        // heads of the tile past the group read as zeros
        const int nvh = hpg - tig * HPT < HPT ? hpg - tig * HPT : HPT;
        const size_t off = (((size_t)b * nc + c) * H + head0) * Q;
        const __amdgpu_buffer_rsrc_t rdt = make_rsrc(a.dtf + off, (uint32_t)(nvh * Q * 4));
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.acs + off, (uint32_t)(nvh * Q * 4));
        for (int e = tid; e < HPT * Q; e += 256) {
            const int hh = e / Q, i = e - hh * Q;
            sDt[hh * QMAX + i] = bload_f32<AUX>(rdt, (uint32_t)e * 4);
            sAcs[hh * QMAX + i] = bload_f32<AUX>(ra, (uint32_t)e * 4);
        }
        if constexpr (varlen) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.seg + ((size_t)b * nc + c) * Q, (uint32_t)Q * 4);
            for (int e = tid; e < Q; e += 256) sSeg[e] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, e * 4, 0, AUX);
        }
    }
    __syncthreads();
    // chunk-state weights; with packed input only the chunk's last sequence reaches its end
    for (int e = tid; e < HPT * Q; e += 256) {
        const int hh = e / Q, i = e - hh * Q;
        const float w = __expf(sAcs[hh * QMAX + Q - 1] - sAcs[hh * QMAX + i]) * sDt[hh * QMAX + i];
        sW[hh * QMAX + i] = (varlen && sSeg[i] != sSeg[Q - 1]) ? 0.f : w;
    }
    const float acs_last = sAcs[hs * QMAX + Q - 1];
    // the state entering the chunk survives to its end unless a sequence starts inside it
    const bool carry = !varlen || sSeg[Q - 1] == 0;

    // S_c in accumulator layout: tile (nb, pb), lane -> S[p = ph*PW + pb*16 + r16][n = nb*16 + 4q + r]
    f32x4 sc[NB][MBP];

    if constexpr (MODE != MODE_SCAN) {
        f32x4 acc[NB][MBP];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb) acc[nb][pb] = vzero<f32x4>();
        T* sBT = (T*)smem;
        T* sXW = (T*)(smem + G_::SZ_BT);
        for (int j0 = 0; j0 < Q; j0 += W) {
            __syncthreads();  // sW ready / previous window's MFMAs done
            stage_transposed<T, N, W, LDW>(sBT, Bg + ((size_t)b * L * Gn + g) * N, (size_t)Gn * N, tok0 + j0, L,
                                           nullptr, tid, 256);
            for (int hh = 0; hh < HPT; ++hh) {
                const bool ok = (tig * HPT + hh) < hpg;
                stage_transposed<T, P, W, LDW>(sXW + hh * P * LDW,
                                               ok ? xg + ((size_t)b * L * H + head0 + hh) * P : nullptr,
                                               (size_t)H * P, tok0 + j0, L, sW + hh * QMAX + j0, tid, 256);
            }
            __syncthreads();
            if (hvalid) {
                const T* xw = sXW + (hs * P + ph * PW) * LDW;
#pragma unroll
                for (int kk = 0; kk < W / KI; ++kk) {
                    frag bfr[MBP];
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) bfr[pb] = load_frag<T>(xw + (pb * 16 + r16) * LDW + kk * KI + q * KPL);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const frag af = load_frag<T>(sBT + (nb * 16 + r16) * LDW + kk * KI + q * KPL);
#pragma unroll
                        for (int pb = 0; pb < MBP; ++pb) acc[nb][pb] = TT<T>::mma(af, bfr[pb], acc[nb][pb]);
                    }
                }
            }
        }
        if constexpr (MODE == MODE_STATE) {
            if (hvalid) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) {
                        const int p = ph * PW + pb * 16 + r16, n = nb * 16 + 4 * q;
                        *(f32x4*)(a.s + ((((size_t)b * nc + c) * H + h) * P + p) * N + n) = acc[nb][pb];
                    }
            }
            return;
        } else if (a.relay && relay_live) {
            // relay form: s_c to the chain's relay item, S_c back
            if (hvalid) relay_handoff<T, NB, MBP>(a, b, c, h, ph, WPH, acc, sc);
        } else {
            // state_passing hop: S_{c+1} = exp(acs[Q-1]) S_c + s_c (a relay-form launch whose
            // partition runs no relay items: counter from 0, the state in the final-state slot 1)
            if (hvalid) {
                uint32_t* fl = chain_counter(a, b, h, ph, WPH);
                const uint32_t base = a.relay ? 0u : 1u;
                wait_flag(fl, a, (uint32_t)c + base);
                const int K = a.slots;
                const int sin = a.relay ? (c > 0 ? 1 : 0) : c % K, sout = a.relay ? 1 : (c + 1) % K;
                const __amdgpu_buffer_rsrc_t rin =
                    ring_rsrc(a.states, a.state_dtype, ring_chain(b, sin, h, ph, K, H, WPH, NB * MBP), NB * MBP);
                const __amdgpu_buffer_rsrc_t rout =
                    ring_rsrc(a.states, a.state_dtype, ring_chain(b, sout, h, ph, K, H, WPH, NB * MBP), NB * MBP);
                const float dec = carry ? __expf(acs_last) : 0.f;
                const bool zero0 = c == 0 && !a.has_h0;  // S_0 = 0: nothing to read
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) {
                        const uint32_t off = ((nb * MBP + pb) * 64 + lane) * 4;
                        sc[nb][pb] = zero0 ? vzero<f32x4>() : ring_load(rin, a.state_dtype, off);
                        ring_store(rout, a.state_dtype, off, dec * sc[nb][pb] + acc[nb][pb]);
                    }
                publish_flag_wave(fl, (uint32_t)c + 1 + base);
            }
        }
    } else {
        if (hvalid) {
            const int K = a.slots, slot = c % K;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int pb = 0; pb < MBP; ++pb) {
                    const int p = ph * PW + pb * 16 + r16, n = nb * 16 + 4 * q;
                    sc[nb][pb] = load_state4(a.states, a.state_dtype, ((((size_t)b * K + slot) * H + h) * P + p) * N + n);
                }
        }
    }

    if constexpr (MODE != MODE_STATE) {
        // ---- chunk_scan ----
        T* sC = (T*)smem;
        T* sL = (T*)(smem + G_::SZ_C);
        T* sXT = (T*)(smem + G_::SZ_C + G_::SZ_L);
        const float Dh = (a.D && hvalid) ? a.D[h] : 0.f;
        const __amdgpu_buffer_rsrc_t rcb = make_rsrc(cbase, (uint32_t)(Q * Q * 4));
        for (int i0 = 0; i0 < Q; i0 += W) {
            __syncthreads();
            stage_rows<T, N, W, LDN>(sC, Cg + ((size_t)b * L * Gn + g) * N, (size_t)Gn * N, tok0 + i0, L);
            __syncthreads();
            f32x4 accY[MBP][WB];
#pragma unroll
            for (int pb = 0; pb < MBP; ++pb)
#pragma unroll
                for (int ib = 0; ib < WB; ++ib) accY[pb][ib] = vzero<f32x4>();
            if (hvalid) {
                // y_off^T[p][i] = sum_n S_c[p][n] C[i][n]: A from the state held in
                // accumulator layout, B from C rows, with matching k-slot order.
                if constexpr (KPL == 8) {
#pragma unroll
                    for (int ks = 0; ks < N / 32; ++ks) {
                        frag af[MBP];
#pragma unroll
                        for (int pb = 0; pb < MBP; ++pb) {
                            const v4 lo = cvt4<T>(sc[2 * ks][pb]);
                            const v4 hi = cvt4<T>(sc[2 * ks + 1][pb]);
                            af[pb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        }
#pragma unroll
                        for (int ib = 0; ib < WB; ++ib) {
                            const T* crow = sC + (ib * 16 + r16) * LDN + ks * 32 + 4 * q;
                            const v4 lo = *(const v4*)crow;
                            const v4 hi = *(const v4*)(crow + 16);
                            const frag bf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                            for (int pb = 0; pb < MBP; ++pb) accY[pb][ib] = TT<T>::mma(af[pb], bf, accY[pb][ib]);
                        }
                    }
                } else {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
#pragma unroll
                            for (int ib = 0; ib < WB; ++ib) {
                                const frag bf = sC[(ib * 16 + r16) * LDN + nb * 16 + 4 * q + r];
#pragma unroll
                                for (int pb = 0; pb < MBP; ++pb)
                                    accY[pb][ib] = TT<T>::mma(sc[nb][pb][r], bf, accY[pb][ib]);
                            }
                }
#pragma unroll
                for (int ib = 0; ib < WB; ++ib) {
                    const int i = i0 + ib * 16 + r16;  // S_c reaches row i only inside the chunk's first sequence
                    const float e = (varlen && sSeg[i] != 0) ? 0.f : __expf(sAcs[hs * QMAX + i]);
#pragma unroll
                    for (int pb = 0; pb < MBP; ++pb) accY[pb][ib] *= e;
                }
            }
            for (int j0 = 0; j0 <= i0; j0 += W) {
                if (j0 > 0) __syncthreads();
                for (int hh = 0; hh < HPT; ++hh) {
                    const bool ok = (tig * HPT + hh) < hpg;
                    stage_transposed<T, P, W, LDW>(sXT + hh * P * LDW,
                                                   ok ? xg + ((size_t)b * L * H + head0 + hh) * P : nullptr,
                                                   (size_t)H * P, tok0 + j0, L, nullptr, tid, 256);
                }
                // L[i][j] = CB[i][j] exp(acs_i - acs_j) dt_j for j <= i in i's sequence, else 0
                // (log-space decay differences in fp32, [HW] segsum section, [XLA] 2.2)
                for (int it = tid; it < W * (W / 4); it += 256) {
                    const int jq = it % (W / 4), ii = it / (W / 4);
                    const int i = i0 + ii, j = j0 + 4 * jq;
                    const f32x4 cbv = bload_f32x4<AUX>(rcb, (uint32_t)(i * Q + j) * 4);
#pragma unroll
                    for (int hh = 0; hh < HPT; ++hh) {
                        const float ai = sAcs[hh * QMAX + i];
                        f32x4 lv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = cbv[e] * __expf(ai - sAcs[hh * QMAX + j + e]) * sDt[hh * QMAX + j + e];
                            const bool same = !varlen || sSeg[i] == sSeg[j + e];
                            lv[e] = (j + e <= i && same) ? v : 0.f;
                        }
                        *(v4*)(sL + (hh * W + ii) * LDW + 4 * jq) = cvt4<T>(lv);
                    }
                }
                __syncthreads();
                if (hvalid) {
                    const T* xt = sXT + (hs * P + ph * PW) * LDW;
                    const T* lt = sL + hs * W * LDW;
#pragma unroll
                    for (int kk = 0; kk < W / KI; ++kk) {
                        frag af[MBP];
#pragma unroll
                        for (int pb = 0; pb < MBP; ++pb) af[pb] = load_frag<T>(xt + (pb * 16 + r16) * LDW + kk * KI + q * KPL);
#pragma unroll
                        for (int ib = 0; ib < WB; ++ib) {
                            if (j0 == i0 && kk * KI > ib * 16 + 15) continue;  // block above the diagonal
                            const frag bf = load_frag<T>(lt + (ib * 16 + r16) * LDW + kk * KI + q * KPL);
#pragma unroll
                            for (int pb = 0; pb < MBP; ++pb) accY[pb][ib] = TT<T>::mma(af[pb], bf, accY[pb][ib]);
                        }
                    }
                }
            }
            if (hvalid) {
                T* yg = (T*)a.y;
#pragma unroll
                for (int ib = 0; ib < WB; ++ib) {
                    const int t = tok0 + i0 + ib * 16 + r16;
                    if (t < L) {
#pragma unroll
                        for (int pb = 0; pb < MBP; ++pb) {
                            const int p = ph * PW + pb * 16 + 4 * q;
                            const size_t off = (((size_t)b * L + t) * H + h) * P + p;
                            const v4 xv = *(const v4*)(xg + off);
                            f32x4 yv = accY[pb][ib];
                            yv[0] += Dh * (float)xv[0];
                            yv[1] += Dh * (float)xv[1];
                            yv[2] += Dh * (float)xv[2];
                            yv[3] += Dh * (float)xv[3];
                            *(v4*)(yg + off) = cvt4<T>(yv);
                        }
                    }
                }
            }
        }
    }
}

}  // namespace ssd
