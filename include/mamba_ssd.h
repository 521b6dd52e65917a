/*
 * mamba_ssd.h -- C ABI of libmamba_ssd.so: the Mamba-2 SSD (state space duality)
 * chunked prefill forward on AMD MI355X (gfx950).
 *
 * What it computes ("Mamba-2状态空间模型的编译器优化与实现", section 1.1, with the
 * Mamba-2 input term): for every batch row b and head h, over t = 0 .. L-1,
 *
 *     dt_t = softplus(dt_raw[b,t,h] + dt_bias[h])            (dt_softplus = 1)
 *     S    = exp(dt_t * A[h]) * S + dt_t * x[b,t,h,:] (outer) B[b,t,g,:]      S is [P, N]
 *     y[b,t,h,:] = S . C[b,t,g,:] + D[h] * x[b,t,h,:]
 *
 * starting from S = initial_state[b,h] (or 0) and ending with final_state[b,h] = S.
 * Head h reads B/C group g = h / (H / G).  The library evaluates it with the chunked
 * algorithm ("Mamba 硬件感知算法", section "块分解与状态传递"; the five steps of
 * "Mamba-2炸裂升级！…", section "Mamba-2核心操作与融合的必要性"): chunk_cumsum, bmm,
 * chunk_state, state_passing, chunk_scan, either as five kernels (SSD_IMPL_UNFUSED)
 * or as one kernel whose workgroups claim cumsum and bmm work first and then
 * chunk_state -> state_passing -> chunk_scan work, ordered by flags and counters
 * (SSD_IMPL_FUSED; same write-up, section "高效内核融合技术揭秘").
 *
 * Conventions for every entry point:
 *   - every tensor pointer is a DEVICE pointer to a contiguous row-major array
 *     owned by the caller; the library never allocates, frees or keeps them;
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream); all
 *     GPU work is enqueued on it asynchronously and nothing synchronises, except
 *     ssd_check_device_status;
 *   - arguments are validated on the host before any HIP call; a failed check
 *     returns an error status and enqueues nothing;
 *   - the library never aborts or throws across this ABI;
 *   - calls are thread-safe; two calls in flight at once need distinct workspaces.
 */
#ifndef MAMBA_SSD_H
#define MAMBA_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 2

/* Element types.  x, dt, B, C and y share `in_dtype`; initial_state, final_state
 * and the inter-chunk states use `state_dtype`; A, D and dt_bias are always fp32. */
typedef enum { SSD_F32 = 0, SSD_F16 = 1, SSD_BF16 = 2 } ssd_dtype_t;

typedef enum { SSD_IMPL_UNFUSED = 0, SSD_IMPL_FUSED = 1 } ssd_impl_t;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    SSD_ERR_INVALID_SHAPE = 2,       /* a size is < 1, or nheads % ngroups != 0, or an index would overflow */
    SSD_ERR_UNSUPPORTED = 3,         /* a legal but unsupported headdim / dstate / chunk_size / dtype combination */
    SSD_ERR_MISALIGNED = 4,          /* a pointer breaks the alignment rule below */
    SSD_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes < ssd_prefill_workspace_size() */
    SSD_ERR_HIP = 6,                 /* a HIP runtime call or kernel launch failed */
    SSD_ERR_SYNC_TIMEOUT = 7,        /* fused kernel: a cross-workgroup wait hit its spin limit (results invalid) */
    SSD_ERR_INVALID_ARGUMENT = 8,    /* an enum field is out of range, or struct_size is too small */
    SSD_ERR_SCHEDULE = 9,            /* fused kernel: a work partition found no workgroup on its XCD (results invalid) */
    SSD_ERR_SCRATCH_TOO_SMALL = 10   /* ssd_prefill_noalloc: the problem's workspace exceeds the static scratch */
} ssd_status_t;

/* Problem description.  Set struct_size = sizeof(ssd_params_t).  A caller built against ABI
 * version 1 passes the smaller struct_size offsetof(ssd_params_t, relaxed) and gets the
 * version-1 behaviour (relaxed = 0). */
typedef struct {
    size_t struct_size;
    int batch;        /* B  >= 1 */
    int seqlen;       /* L  >= 1; need not be a multiple of chunk_size (the last chunk is masked) */
    int nheads;       /* H  >= 1 */
    int headdim;      /* P in {16, 32, 64, 128} */
    int dstate;       /* N in {32, 64, 128} (also 16 when in_dtype is SSD_F32) */
    int ngroups;      /* G >= 1, H % G == 0 */
    int chunk_size;   /* Q in {64, 128, 256} */
    int in_dtype;     /* ssd_dtype_t */
    int state_dtype;  /* ssd_dtype_t */
    int dt_softplus;  /* 1: dt = softplus(dt_raw + dt_bias); 0: dt = dt_raw + dt_bias */
    int impl;         /* ssd_impl_t */
    /* ABI version 2: */
    int relaxed;      /* 0: exact intermediates; 1: relaxed ("Mamba-2炸裂升级！…", section
                         "精度与性能的平衡艺术"): with 16-bit inputs CB = C B^T of each chunk is
                         stored in in_dtype instead of fp32 (no effect for fp32 inputs) */
    int flags;        /* 0, or SSD_FLAG_WORKSPACE_READY (below); other bits must be 0 */
} ssd_params_t;

/* flags bit 0 (fused form; ignored by the unfused form and by ssd_prefill_block): the
 * workspace's synchronisation words are as the previous fused call on this workspace left them,
 * and that call had the same parameters (every field but flags) and ran in this process.  Every
 * fused call that writes a final_state resets those words for the next call in the launch that
 * copies the final state out, so a caller that reuses one workspace for a run of identical calls
 * sets this bit on all but the first: a call without an initial state then skips the launch that
 * would reset them (one launch fewer per call).  The library keeps, per workspace address, the
 * parameters of the last call that left it ready; when they differ, or the last call on the
 * workspace was not such a call, the bit is ignored and the words are reset as usual.  A caller
 * who wrote to the workspace in between, or freed and re-allocated it, must not set the bit.
 * As with any reuse of one workspace, the calls must be ordered on the device (one stream, or
 * the earlier call complete before the later one starts).
 * The device status word (ssd_check_device_status) is cleared only by a call that resets the
 * words: after an error, calls with this bit keep reporting it until a call without the bit. */
#define SSD_FLAG_WORKSPACE_READY 1

/*
 * Tensor arguments (all device pointers):
 *   x             [B, L, H, P]  in_dtype     required, 16-byte aligned
 *   dt            [B, L, H]     in_dtype     required (raw step, before bias / softplus)
 *   A             [H]           fp32         required; A <= 0 is a precondition (not checked;
 *                                            A = 0 gives causal linear attention)
 *   (dt)                                     with dt_softplus = 0 the step dt_raw + dt_bias may
 *                                            have either sign (a negative step grows the state,
 *                                            as the recurrence says); every decay is evaluated as
 *                                            exp of a difference of fp32 in-chunk sums of dt * A,
 *                                            so those sums must stay within about +-87 over any
 *                                            chunk when some dt * A > 0 (fp32 exp range)
 *   B, C          [B, L, G, N]  in_dtype     required, 16-byte aligned
 *   D             [H]           fp32         NULL means 0
 *   dt_bias       [H]           fp32         NULL means 0
 *   initial_state [B, H, P, N]  state_dtype  NULL means 0; 16-byte aligned
 *   y             [B, L, H, P]  in_dtype     required output, 16-byte aligned
 *   final_state   [B, H, P, N]  state_dtype  required output, 16-byte aligned
 *   workspace     bytes         -            required, 256-byte aligned, at least
 *                                            ssd_prefill_workspace_size() bytes; its contents
 *                                            need no initialisation and are overwritten
 *                                            (but see SSD_FLAG_WORKSPACE_READY)
 */

/* Bytes of workspace ssd_prefill needs for *p (0 if *p is invalid: see ssd_validate). */
size_t ssd_prefill_workspace_size(const ssd_params_t* p);

/* Host-only check of *p (shape, support and enum rules above).  Makes no HIP call. */
ssd_status_t ssd_validate(const ssd_params_t* p);

/* One SSD prefill: y and final_state from the inputs, enqueued on `stream`. */
ssd_status_t ssd_prefill(const ssd_params_t* p,
                         const void* x, const void* dt, const float* A,
                         const void* B, const void* C,
                         const float* D, const float* dt_bias,
                         const void* initial_state,
                         void* y, void* final_state,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ssd_prefill plus timing: records the caller's HIP events `kernel_begin` and
 * `kernel_end` (hipEvent_t passed as void*, both required, created by the caller) on
 * `stream` immediately before and after the SSD compute kernels -- the single fused
 * kernel for SSD_IMPL_FUSED; the five step kernels (with the state-passing boundary
 * copies between them) for SSD_IMPL_UNFUSED -- so their elapsed time excludes the
 * fused form's boundary copies.  Same arguments and errors as ssd_prefill otherwise. */
ssd_status_t ssd_prefill_timed(const ssd_params_t* p,
                               const void* x, const void* dt, const float* A,
                               const void* B, const void* C,
                               const float* D, const float* dt_bias,
                               const void* initial_state,
                               void* y, void* final_state,
                               void* workspace, size_t workspace_bytes, void* stream,
                               void* kernel_begin, void* kernel_end);

/* Packed variable-length input ("Mamba-2炸裂升级！…", section "与vLLM的深度融合":
 * several sequences share a batch row without padding and are told apart by a per-token
 * sequence index, handled by masking).  Same as ssd_prefill, plus
 *   seq_idx  [B, L]  int32  required, 4-byte aligned: a new sequence starts at every t > 0
 *                           with seq_idx[b,t] != seq_idx[b,t-1]; the recurrence restarts
 *                           there from S = 0.
 * Each batch row's initial_state is the state entering its first sequence, and
 * final_state[b] is the state after token L-1 (of its last sequence); sequences in the
 * middle of a row start from zero and their end states are not written out.  The
 * chunk_cumsum step counts the sequence starts inside each chunk (workspace `seg`) and every
 * later step masks with those counts: a decay between two tokens is used only when both lie
 * in one sequence, the state entering a chunk only reaches the tokens before the chunk's
 * first sequence start, and a chunk with a start inside passes on only its last sequence's
 * state.  The in-chunk log-decay sums are those of the unpacked input, so packing costs no
 * precision. */
ssd_status_t ssd_prefill_varlen(const ssd_params_t* p,
                                const void* x, const void* dt, const float* A,
                                const void* B, const void* C,
                                const float* D, const float* dt_bias,
                                const int32_t* seq_idx,
                                const void* initial_state,
                                void* y, void* final_state,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Packed variable-length input with a state per sequence (the same section of the kernel-fusion
 * write-up: variable-length sequences and their initial states without padding, one pseudo-chunk
 * per sequence in a chunk, handled by masking).  Same as ssd_prefill_varlen except:
 *   - a sequence starts at t = 0 of every row as well as wherever seq_idx changes, and
 *     seq_idx[b,t] in [0, nseq) is the number of the sequence holding token t; each number
 *     labels one run of tokens (a number used by two runs gets either run's final state);
 *   initial_states [nseq, H, P, N] state_dtype  NULL means 0; 16-byte aligned: sequence q starts
 *                                               from initial_states[q];
 *   final_states   [nseq, H, P, N] state_dtype  required output, 16-byte aligned: the state after
 *                                               the last token of sequence q; entries of numbers
 *                                               no run uses are left as they were.
 * There is no per-row initial or final state.  Tokens whose number lies outside [0, nseq) run
 * from a zero state and write no final state.  16-bit inputs only (fp32: SSD_ERR_UNSUPPORTED);
 * the fused form hands states over in its chunk tiles (no relay items).  nseq < 1:
 * SSD_ERR_INVALID_SHAPE. */
ssd_status_t ssd_prefill_varlen_states(const ssd_params_t* p,
                                       const void* x, const void* dt, const float* A,
                                       const void* B, const void* C,
                                       const float* D, const float* dt_bias,
                                       const int32_t* seq_idx, int nseq,
                                       const void* initial_states,
                                       void* y, void* final_states,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* ssd_prefill without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a static device array inside the library, SSD_NOALLOC_SCRATCH_BYTES bytes on each
 * GPU the library runs on, held until the process ends; its address on the current device is
 * looked up once per device, on that device's first call.  The call allocates nothing and makes
 * no allocating library call.  Arguments, layouts and errors are ssd_prefill's, plus
 *   SSD_ERR_SCRATCH_TOO_SMALL  when ssd_prefill_workspace_size(p) > SSD_NOALLOC_SCRATCH_BYTES
 *                              (nothing is enqueued);
 *   SSD_ERR_HIP                when the scratch's address cannot be obtained.
 * Every call on one GPU uses the same scratch, which keeps the previous call's contents (each
 * call resets what must start at zero with a kernel): calls that overlap in time on one GPU
 * (different streams, or different host threads) race and give wrong results; serialise them.
 * The device status of such a call (SSD_ERR_SYNC_TIMEOUT / SSD_ERR_SCHEDULE) is not readable:
 * ssd_check_device_status needs the workspace, so diagnose with ssd_prefill. */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)320 << 20)
ssd_status_t ssd_prefill_noalloc(const ssd_params_t* p,
                                 const void* x, const void* dt, const float* A,
                                 const void* B, const void* C,
                                 const float* D, const float* dt_bias,
                                 const void* initial_state,
                                 void* y, void* final_state, void* stream);

/* Synchronises `stream`, then reads the device status word the last fused
 * ssd_prefill on `workspace` left: SSD_OK, SSD_ERR_SYNC_TIMEOUT when one of its waits
 * gave up, or SSD_ERR_SCHEDULE when one of its work partitions was never served (in
 * both cases its outputs are invalid).  SSD_ERR_HIP if a HIP call fails. */
ssd_status_t ssd_check_device_status(const ssd_params_t* p, const void* workspace, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* ssd_status_string(ssd_status_t s);

/* ------------------------------------------------------------------------------------
 * Workspace layout, for the per-step entry points below and for tests that read the
 * intermediates.  Offsets are in bytes from the workspace start; nc = ceil(L / Q).
 *   dt      fp32 [B][nc][H][Q]       step size per token (0 past seqlen)       chunk_cumsum
 *   acs     fp32 [B][nc][H][Q]       inclusive in-chunk sum of dt * A            chunk_cumsum
 *   cb      fp32 [B][nc][G][Q][Q]    CB[i][j] = C_i . B_j for j <= i; entries
 *                                    with j > i are never written nor read      bmm
 *           fused: [B*G + 7][nc][Q][Q], one [nc] run per (work partition, (b, g) pair)
 *   s       fp32 [B][nc][H][P][N]    chunk-end state from a zero start            chunk_state
 *           unfused: as shown; fused: 0 bytes, or with the relay form's buffers (below) a
 *           ring of 10 chunk states per chain ([B][H][P][N] x 10 fp32) followed by a ring of
 *           min(6, nc + 1) states in in_dtype ([B][H][P][N] x min(6, nc + 1)), both in the
 *           fused kernel's own order
 *   states  state_dtype, K slots     state entering chunk c lives in slot c % K; slot 0
 *                                    holds the initial state, slot nc % K the final one
 *           unfused: [B][K = nc+1][H][P][N]                                      state_passing
 *           fused:   K = 1 slot per chain, updated in place chunk after chunk (relay form:
 *                    K = 2, the initial state in slot 0 and the final one in slot 1), in an
 *                    internal lane-major order (the fused kernel's own layout); without an
 *                    initial state slot 0 is not filled (the kernel takes S_0 = 0)
 *   seg     int32 [B][nc][Q]         packed input (ssd_prefill_varlen) only: the number of
 *                                    sequence starts among chunk tokens 0 .. i   chunk_cumsum
 *   sync    uint32 words: per-chain words (three 128-byte lines each: progress counter,
 *           relay slot words), cumsum / bmm completion flags, one work counter per
 *           partition, then per partition an owner word, a count of the workgroups that
 *           joined it and its relay decision, the exit counter and the abort word (fused only)
 *   status  uint32 device status word
 * The fused form splits its work into one partition per XCD of the device (at most 8);
 * the sizes above are bounds that hold for any such split.  Shapes with at most 128
 * chains (batch * ngroups * ceil(heads per group / heads per tile); 4 heads per tile
 * for headdim <= 32, 2 for 64, 1 for 128) get the buffers of the fused relay form, in which
 * dedicated work items (2 or 4 per chain) pass the state from chunk to chunk; it is used
 * when they take at most half of the workgroups a partition holds at once (the fused
 * kernel's occupancy times the XCD's compute units), and each partition checks that rule
 * again on the device against the workgroups that actually joined it, its chunk tiles
 * passing the state themselves where it fails.  The environment variable MAMBA_SSD_RELAY =
 * 0 / 1 forces the buffers off / on (2 / 4: on, with that many items per chain); it is read
 * on every call, so workspace sizing and the call must see the same value.
 * Test knobs, also read on every call: MAMBA_SSD_SPIN_LIMIT (polls before a wait gives up),
 * MAMBA_SSD_RELAY_ADMIT=0 (every partition refuses its relay items) and
 * MAMBA_SSD_GRID_LIMIT (caps the fused grid; unserved partitions give SSD_ERR_SCHEDULE).
 * ------------------------------------------------------------------------------------ */
typedef struct {
    size_t total_bytes;
    size_t dt_offset, acs_offset, cb_offset, s_offset, states_offset, sync_offset, status_offset;
    size_t dt_bytes, acs_bytes, cb_bytes, s_bytes, states_bytes, sync_bytes;
    int nchunks;
    int state_slots;  /* K */
    size_t seg_offset, seg_bytes;
} ssd_workspace_layout_t;

ssd_status_t ssd_workspace_layout(const ssd_params_t* p, ssd_workspace_layout_t* out);

/* ------------------------------------------------------------------------------------
 * The five steps of the unfused form, one entry point each, with the same argument
 * rules as ssd_prefill (p->impl must be SSD_IMPL_UNFUSED).  Each reads the workspace
 * intermediates the previous steps wrote and writes its own.  Calling them in this
 * order equals ssd_prefill with impl = SSD_IMPL_UNFUSED.
 * ------------------------------------------------------------------------------------ */

/* chunk_cumsum ("Mamba-2炸裂升级！…", section "Mamba-2核心操作与融合的必要性", item 4):
 * per-token dt and its in-chunk cumulative decay -> workspace dt, acs. */
ssd_status_t ssd_step_chunk_cumsum(const ssd_params_t* p, const void* dt, const float* A,
                                   const float* dt_bias, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* bmm (same section, item 7): CB = C B^T inside each chunk and group -> workspace cb. */
ssd_status_t ssd_step_bmm(const ssd_params_t* p, const void* B, const void* C,
                          void* workspace, size_t workspace_bytes, void* stream);

/* chunk_state (item 5): each chunk's end state from a zero start, the decay to the
 * chunk end applied to x (same write-up, section "性能瓶颈的深入分析") -> workspace s. */
ssd_status_t ssd_step_chunk_state(const ssd_params_t* p, const void* x, const void* B,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* state_passing (item 6): copies initial_state into slot 0, runs
 * S_{c+1} = exp(acs_c[Q-1]) S_c + s_c over the chunks, copies the last slot to
 * final_state (the boundary split-out of section "性能瓶颈的深入分析"). */
ssd_status_t ssd_step_state_passing(const ssd_params_t* p, const void* initial_state,
                                    void* final_state, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* chunk_scan (item 8): y from x, C, the chunk-entry states and CB -> y. */
ssd_status_t ssd_step_chunk_scan(const ssd_params_t* p, const void* x, const void* C,
                                 const float* D, void* y, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ------------------------------------------------------------------------------------
 * Single-token decode step ("Mamba-2状态空间模型的编译器优化与实现", section 2.1: the
 * cache holds the [B,H,P,N] SSM state and each generated token applies the recurrence
 * once; section 3.2: the step is bound by memory bandwidth and runs as one pass over
 * HBM).  It is exactly one token of the recurrence at the top of this header, started
 * from state_in and ending in state_out:
 *
 *     dt = softplus(dt_raw[b,h] + dt_bias[h])   (dt_softplus = 1)
 *     S  = exp(dt * A[h]) * state_in[b,h] + dt * x[b,h,:] (outer) B[b,g,:]
 *     y[b,h,:] = S . C[b,g,:] + D[h] * x[b,h,:],   state_out[b,h] = S   (g = h / (H / G))
 *
 * so ssd_prefill of L tokens followed by ssd_decode_step on the next tokens, each
 * taking the previous final state, equals ssd_prefill of the longer sequence.
 *
 * Parameters: *p as for ssd_prefill except that p->seqlen must be 1 (one token per
 * batch row; SSD_ERR_INVALID_SHAPE otherwise), p->headdim may be any P >= 1, p->dstate
 * must be one of 16, 32, 64, 128, 256 (SSD_ERR_UNSUPPORTED otherwise), and chunk_size
 * and impl are ignored.
 *
 * Tensor arguments (device pointers; the layouts are ssd_prefill's with L = 1):
 *   x          [B, H, P]     in_dtype     required, 16-byte aligned
 *   dt         [B, H]        in_dtype     required (raw step, before bias / softplus)
 *   A          [H]           fp32         required (A <= 0, not checked)
 *   B, C       [B, G, N]     in_dtype     required, 16-byte aligned
 *   D, dt_bias [H]           fp32         NULL means 0
 *   state_in   [B, H, P, N]  state_dtype  NULL means 0; 16-byte aligned
 *   state_out  [B, H, P, N]  state_dtype  required, 16-byte aligned; may be the same
 *                                         buffer as state_in (in-place update); any other
 *                                         overlap with state_in is undefined
 *   y          [B, H, P]     in_dtype     required output, 16-byte aligned
 * The update runs in fp32 and rounds the state to state_dtype once.  No workspace, no
 * allocation, no synchronisation; one kernel on `stream`.  Errors as for ssd_prefill
 * (validated on the host before the launch). */
ssd_status_t ssd_decode_step(const ssd_params_t* p,
                             const void* x, const void* dt, const float* A,
                             const void* B, const void* C,
                             const float* D, const float* dt_bias,
                             const void* state_in, void* state_out, void* y, void* stream);

/* ---- The Mamba-2 block around the SSD ------------------------------------------------------
 * The operations just before and after the SSD in a Mamba-2 block ("Mamba-2炸裂升级！…", section
 * "Mamba-2核心操作与融合的必要性": the depthwise convolution over the last few tokens; section
 * "未来展望与应用拓展": fusing the convolution before and the norm after the SSD into its launch,
 * each saving a full write and read of an activation).  16-bit inputs only (fp32:
 * SSD_ERR_UNSUPPORTED).  With Ch = H*P + 2*G*N channels:
 *   xbc        [B, L, Ch]    in_dtype  required, 16-byte aligned: the SSD's inputs before the
 *                                      convolution, channels [x (h*P + p) | B (g*N + n) | C (g*N + n)]
 *   conv_w     [Ch, 4]       fp32      required, 16-byte aligned: the taps of the causal depthwise
 *                                      convolution of width 4
 *   conv_b     [Ch]          fp32      NULL means 0
 *   conv_state [B, Ch, 3]    in_dtype  NULL means 0: the 3 inputs before token 0 (a decode
 *                                      cache's convolution state)
 * and the convolution is x, B, C = silu(conv_b + sum_k conv_w[:, k] * xbc[t - 3 + k]), rounded to
 * in_dtype.  The norm after the SSD is Mamba-2's gated RMS norm with one group per B/C group:
 *   z          [B, L, H*P]   in_dtype  required, 16-byte aligned
 *   norm_w     [H*P]         fp32      required, 16-byte aligned
 *   out[b,t,c] = g / sqrt(mean over the H/G*P channels of c's group of g^2 + norm_eps) * norm_w[c],
 *                g = y[b,t,c] * silu(z[b,t,c]);  norm_eps >= 0 (else SSD_ERR_INVALID_ARGUMENT).
 */

/* The convolution alone: xbc -> x [B, L, H, P], B and C [B, L, G, N] (16-byte aligned). */
ssd_status_t ssd_conv_silu(const ssd_params_t* p, const void* xbc, const float* conv_w, const float* conv_b,
                           const void* conv_state, void* x, void* B, void* C, void* stream);

/* The gated norm alone: y, z -> out, all [B, L, H*P] in_dtype (16-byte aligned). */
ssd_status_t ssd_gated_norm(const ssd_params_t* p, const void* y, const void* z, const float* norm_w,
                            float norm_eps, void* out, void* stream);

/* Workspace bytes ssd_prefill_block needs (0 if *p is invalid or not 16-bit). */
size_t ssd_prefill_block_workspace_size(const ssd_params_t* p);

/* Convolution, SSD prefill and gated norm: out [B, L, H*P] and final_state [B, H, P, N] from xbc,
 * dt, A, D, dt_bias, z, the initial state and the taps above (arguments as for ssd_prefill and
 * the block section above; workspace 256-byte aligned, at least
 * ssd_prefill_block_workspace_size() bytes).
 *   SSD_IMPL_UNFUSED: the convolution kernel, the five SSD kernels and the norm kernel, with x,
 *     B, C and y going through the workspace.
 *   SSD_IMPL_FUSED: the convolution inside the SSD launch (plus the boundary copies): the bmm
 *     tiles convolve B and C from xbc and the chunk tiles convolve their x rows in LDS; y goes
 *     through the workspace to the norm kernel.  With MAMBA_SSD_BLOCK_NORM=1 the norm runs inside
 *     the launch too, where every (b, g) pair's tiles fall in one work partition (one XCD): the
 *     chunk tiles write y to out with each token's share of the squared sums of y silu(z), and a
 *     norm item per tile, after all chunk tiles in the queue, scales those rows (measured slower
 *     on MI355X than the norm kernel).  headdim and dstate in {64, 128} with H/G a multiple of
 *     the heads per tile (2 at headdim 64), else SSD_ERR_UNSUPPORTED. */
ssd_status_t ssd_prefill_block(const ssd_params_t* p, const void* xbc, const float* conv_w, const float* conv_b,
                               const void* conv_state, const void* dt, const float* A, const float* D,
                               const float* dt_bias, const void* z, const float* norm_w, float norm_eps,
                               const void* initial_state, void* out, void* final_state,
                               void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SSD_H */
