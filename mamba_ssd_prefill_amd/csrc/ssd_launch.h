// ssd_launch.h -- host-side interface between the C-ABI layer and the kernel
// translation units: the kernel argument block and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

// Largest number of XCDs (L2 domains) the fused form partitions its work over.
constexpr int kMaxXcc = 8;

// Kernel argument block (passed by value).  Layouts are described in mamba_ssd.h.
struct SsdArgs {
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* dt_bias;
    const int* seq_idx;  // [B][L] sequence ids of packed variable-length input, or nullptr
    int* seg;            // [B][nc][Q] with seq_idx: sequence starts among chunk tokens 0..i
    void* y;
    float* dtf;          // [B][nc][H][Q]
    float* acs;          // [B][nc][H][Q]
    float* cb;           // unfused: [B][nc][G][Q][Q]; fused: [pair slot][nc][Q][Q]; fp32, or the 16-bit
                         // input type when cb16 (see cb_at)
    float* s;            // unfused: [B][nc][H][P][N]; fused relay form: the chunk-state ring
    void* states;        // unfused: [B][K][H][P][N]; fused: K ring slots per chain
    void* opnd;          // fused relay form: S_c in the operand type, op_slots slots per chain
    uint32_t* flags;     // fused: per-chain words [B][H][WPH], kChainStride words apart
    uint32_t* cs_done;   // fused: [pair slot][nc]
    uint32_t* bmm_done;  // fused: [pair slot][nc]
    uint32_t* ticket;    // fused: one work counter per partition, kTicketStride words apart
    uint32_t* owner;     // fused: [kMaxXcc] hardware XCC id (+1) that serves each partition
    uint32_t* joined;    // fused: [kMaxXcc] workgroups that joined each partition
    uint32_t* relay_on;  // fused relay form: [kMaxXcc] 0 undecided, 1 relay items run, 2 chunk tiles hop
    uint32_t* exit_count;
    uint32_t* abort_word;
    uint32_t* status;
    int batch, seqlen, nheads, ngroups, chunk, nchunks, hpg, tpg, slots, op_slots;
    int state_dtype, softplus;
    int has_h0;  // fused form: 0 = no initial state (S_0 = 0 is never read from the ring)
    uint32_t spin_limit;
    // fused form: the chains (b, g, tile-in-group), numbered u = (b * G + g) * tpg + tig, are
    // split into nparts contiguous ranges [part_u0[x], part_u0[x + 1]); partition x runs on
    // the XCD whose id is x modulo nparts.  Its (b, g) pairs use cb / flag slots starting at
    // part_pb[x].
    int nparts;
    int part_u0[kMaxXcc + 1];
    int part_pb[kMaxXcc + 1];
    int chain_group;    // chains whose chunk tiles are claimed together (0: set at launch)
    int relay;          // fused form: relay waves per chain part (2 or 4), 0 = no relay items
    int relay_admit;    // fused relay form: 0 makes every partition decide "chunk tiles hop" (a test knob)
    int agg16;          // fused relay form: the chunk-state ring holds fp16 (fp16 state storage), else fp32
    int agg_slots;      // fused relay form: chunk-state ring slots per chain part (<= kAggSlots)
    int cb16;           // relaxed intermediates: CB stored in the 16-bit input type instead of fp32
    // packed input with per-sequence states (ssd_prefill_varlen_states): a row's first token
    // starts a sequence too; seq_idx[b][t] in [0, nseq) numbers the sequence, whose initial
    // state is seq_h0[q] (nullptr: zero) and whose final state goes to seq_fin[q], both
    // [nseq][H][P][N] in the state dtype
    int seqstates, nseq;
    const void* seq_h0;
    void* seq_fin;
    // block form (the convolution before and the norm after the SSD in one launch): x is read
    // from xbc [B][L][x_stride] (x_stride = H*P + 2*G*N; x in channels 0 .. H*P - 1, B at
    // xbc_hp + g*N, C at xbc_hp + G*N + g*N) through the width-4 convolution (conv_w [ch][4],
    // conv_b [ch] fp32, conv_state [B][ch][3] or nullptr); the bmm tiles convolve B and C into B
    // and C (workspace, [B][L][G][N]).  With norm_fused the chunk tiles write the gated rows
    // y silu(z) to out instead of y, summing each token's squares in nsum [B][L][G] and counting
    // finished tiles in ncount [B][nc][G]; norm items (norm_ticket) then scale those rows.
    int x_stride;       // elements between the token rows of x (H*P without the block form)
    const void* xbc;
    int xbc_hp;
    const float* conv_w;
    const float* conv_b;
    const void* conv_state;
    int norm_fused;
    const void* z;
    const float* norm_w;
    float norm_eps;
    float* nsum;
    uint32_t* ncount;
    void* out;
    int part_max_work;  // host only: the longest partition queue
    int cu_count;       // host only: compute units of the device
    int fused_occ;      // host only: workgroups of the fused kernel one CU holds at once
};

constexpr int kTicketStride = 32;  // one 128-byte line per partition counter
// Fused form, per chain (b, h, p-slice): three 128-byte lines of sync words -- the progress
// counter, then (relay form) the chunk-state slot words and the state read words.
constexpr int kChainStride = 96;
constexpr int kChainAggWords = 32;
constexpr int kChainReadWords = 64;
// Relay form: operand ring slots and chunk-state ring slots per chain (each at most 32, one
// line of slot words).  Its state ring has two slots: the initial state and the final one.
// Small rings keep a chain's hand-off buffers resident in the XCD's L2 (measured on MI355X:
// 10 and 6 slots beat 32 and 16 by 4-5 % on the relay-form shapes; the chunk tiles run only a
// few chunks ahead of the relay waves anyway).
constexpr int kRelaySlots = 6;
constexpr int kAggSlots = 10;  // chunk-state ring slots per chain part (the most; SsdArgs::agg_slots)
// Long chains (more than kLongChainChunks chunks) get a ring of kAggSlotsLong: measured on
// MI355X, 4 slots against 10 take the 131K-token context from 2.41 to 2.29 ms and the packed
// 32 x 1024-token batch from 1.13 to 1.05 ms, while the 32-chunk 130M layer is 2.5 % slower with
// them (and 3 or 2 slots are slower everywhere).
constexpr int kAggSlotsLong = 4;
constexpr int kLongChainChunks = 64;


enum : int {
    STEP_CUMSUM = 0,
    STEP_BMM = 1,
    STEP_CHUNK_STATE = 2,
    STEP_STATE_PASSING = 3,
    STEP_CHUNK_SCAN = 4,
    STEP_FUSED = 5,
    STEP_FUSED_OCCUPANCY = 6,  // host only: sets SsdArgs::fused_occ for the fused kernel, launches nothing
};

// Relay admission, the same rule on the host (with the workgroups a partition can hold) and on
// the device (with the workgroups that actually joined it): relay items, R per chain, may take at
// most half of the partition's workgroups and must leave room for two chunks of its chunk tiles.
__host__ __device__ inline bool relay_fits(int R, int nu, int workgroups) {
    return 2 * R * nu <= workgroups && workgroups - R * nu >= 2 * nu + 2;
}

// Work split of a chunk tile for headdim P: PW columns of P per wave, WPH waves per
// head, HPT = 4 / WPH heads per 256-thread workgroup.
inline int p_per_wave(int P) { return P < 32 ? P : 32; }
inline int waves_per_head(int P) { return P / p_per_wave(P); }
inline int heads_per_tile(int P) { return 4 / waves_per_head(P); }

// Per-dtype launchers; hipErrorNotSupported when (P, N) has no instantiation.
hipError_t launch_step_f32(int step, int P, int N, SsdArgs& a, hipStream_t st);
hipError_t launch_step_f16(int step, int P, int N, SsdArgs& a, hipStream_t st);
hipError_t launch_step_bf16(int step, int P, int N, SsdArgs& a, hipStream_t st);
// One translation unit per (dtype, chunk size, packed input or not); vl1 = packed input
hipError_t launch_step_f32_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st);
hipError_t launch_step_f32_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st);
#define SSD_DECLARE_16(dt)                                                                 \
    hipError_t launch_step_##dt##_q64_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st);  \
    hipError_t launch_step_##dt##_q64_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st);  \
    hipError_t launch_step_##dt##_q128_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st); \
    hipError_t launch_step_##dt##_q128_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st); \
    hipError_t launch_step_##dt##_q256_vl0(int step, int P, int N, SsdArgs& a, hipStream_t st); \
    hipError_t launch_step_##dt##_q256_vl1(int step, int P, int N, SsdArgs& a, hipStream_t st);
SSD_DECLARE_16(f16)
SSD_DECLARE_16(bf16)
#undef SSD_DECLARE_16

// Argument block of the single-token decode step (ssd_decode.hip); layouts in mamba_ssd.h.
struct DecodeArgs {
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const float* dt_bias;
    const void* state_in;  // nullptr: zero state
    void* state_out;       // may equal state_in
    void* y;
    int batch, nheads, headdim, dstate, ngroups, state_dtype, softplus;
};

// State rows of P one decode workgroup covers (kDecodeIter loads per lane, 256 / N rows each).
// (4 measured fastest on MI355X: 8 or 16 loads per lane were slower)
constexpr int kDecodeIter = 4;
inline int decode_rows_per_block(int N) { return 4 * kDecodeIter * (256 / N); }

// The decode step for dstate N in {16, 32, 64, 128, 256}; hipErrorNotSupported otherwise.
hipError_t launch_decode(DecodeArgs& a, int in_dtype, hipStream_t st);

// The steps around the SSD in the Mamba-2 block (ssd_block.hip), 16-bit inputs only.
// conv: xbc [B][L][hp + 2 gn] -> x [B][L][hp], B and C [B][L][gn] (silu of the causal depthwise
// convolution of width 4; w [ch][4], bias [ch] fp32; state [B][ch][3] or nullptr).
struct ConvArgs {
    const void* xbc;
    const float* w;
    const float* bias;
    const void* state;
    void* x;
    void* B;
    void* C;
    int batch, seqlen, hp, gn;
};
// gated norm over rows tokens: out = y silu(z) / sqrt(mean_group (y silu(z))^2 + eps) * w,
// y, z, out [rows][hp], w [hp] fp32, groups contiguous channel groups of hp / groups.
struct NormArgs {
    const void* y;
    const void* z;
    const float* w;
    void* out;
    int64_t rows;
    int hp, groups;
    float eps;
};
hipError_t launch_conv_silu(ConvArgs& a, int in_dtype, hipStream_t st);
// The fused block form (STEP_FUSED / STEP_FUSED_OCCUPANCY), P and N in {64, 128}.
hipError_t launch_block_f16(int step, int P, int N, int Q, SsdArgs& a, hipStream_t st);
hipError_t launch_block_bf16(int step, int P, int N, int Q, SsdArgs& a, hipStream_t st);
hipError_t launch_gated_norm(NormArgs& a, int in_dtype, hipStream_t st);

// Non-templated kernels (ssd_common.hip).
hipError_t launch_state_passing(SsdArgs& a, int PN, hipStream_t st);
// keep: index of a sync word left as it is (the status word, when the final-state copy resets
// the words for the next call), ~0 for none.
hipError_t launch_ring_copy(const void* src, void* dst, int to_ring, int B, int H, int P, int PW, int N, int K,
                            int slot, int es, int pperm, uint32_t* sync, size_t nsync, size_t nflags,
                            uint32_t flag_period, uint32_t flag_init, size_t keep, hipStream_t st);
hipError_t launch_boundary(const void* src, size_t src_bs, void* dst, size_t dst_bs, size_t bytes_per_b,
                           int batch, uint32_t* sync, size_t nsync, size_t nflags, uint32_t flag_period,
                           hipStream_t st);

}  // namespace ssd
