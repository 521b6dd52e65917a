// ssd_kernels.h -- __global__ entry points of the SSD prefill and their host launchers.
// Included once per input dtype by ssd_kernels_{f32,f16,bf16}.hip, which instantiate
// the launchers for the supported (headdim, dstate) pairs.
#pragma once

#include <stdlib.h>

#include "ssd_device.h"
#include "ssd_tile16.h"

namespace ssd {

// No-op hooks (see ClaimHook) for the unfused kernels.
struct NoHook {
    __device__ inline void claim() const {}
    __device__ inline bool relay_live() const { return false; }
};

// ---- unfused form: one kernel per step -------------------------------------------------
template <typename T> __global__ __launch_bounds__(256) void k_chunk_cumsum(SsdArgs a) {
    const int c = blockIdx.x % a.nchunks, b = blockIdx.x / a.nchunks;
    cumsum_tile<T>(a, b, c, 0, a.nheads);
}

__device__ inline float* cb_global(const SsdArgs& a, int b, int c, int g) {
    return cb_at(a, ((size_t)b * a.nchunks + c) * a.ngroups + g);
}

template <typename T, int N> __global__ __launch_bounds__(256) void k_bmm(SsdArgs a) {
    const int g = blockIdx.x % a.ngroups;
    const int c = (blockIdx.x / a.ngroups) % a.nchunks;
    const int b = blockIdx.x / (a.ngroups * a.nchunks);
    bmm_tile<T, N>(a, b, c, g, cb_global(a, b, c, g));
}

// blockIdx.x -> (b, c, g, tile-in-group).  VL: packed variable-length input (a.seq_idx set).
template <typename T, int P, int N, int MODE, int VL> __global__ __launch_bounds__(256) void k_chunk(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo<T, P, N>::SMEM];
    int r = blockIdx.x;
    const int tig = r % a.tpg;
    r /= a.tpg;
    const int g = r % a.ngroups;
    r /= a.ngroups;
    const int c = r % a.nchunks;
    const int b = r / a.nchunks;
    chunk_tile<T, P, N, MODE, VL>(a, b, c, g, tig, smem, cb_global(a, b, c, g));
}

template <typename T, int P, int N, int Q, int MODE, int VL>
__global__ __launch_bounds__(256) void k_chunk16(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo16<T, P, N, Q>::SMEM];
    int r = blockIdx.x;
    const int tig = r % a.tpg;
    r /= a.tpg;
    const int g = r % a.ngroups;
    r /= a.ngroups;
    const int c = r % a.nchunks;
    const int b = r / a.nchunks;
    chunk_tile16<T, P, N, Q, MODE, VL>(a, b, c, g, tig, smem, cb_global(a, b, c, g), NoHook{});
}

// ---- fused form: a single launch ([KF] "高效内核融合技术揭秘") ------------------------------
// The chains u = (b, g, tile-in-group) are split into contiguous partitions, one per XCD.
// Partition x owns the chunk tiles (u, c) of its chains and its own copy of the cumsum and
// bmm work those tiles read: cumsum tiles (pair, c) over the heads of its chains in pair
// (b, g), and bmm tiles (pair, c) into its own CB slots.  Its queue, in claim order:
//   [0, np*nc)             cumsum tiles, chunk-major
//   [np*nc, 2*np*nc)       bmm tiles, chunk-major
//   [2*np*nc, +R*nu)       relay form only: R relay items per chain (R = relay waves per part,
//                          2 or 4), each serving 4 / R parts of it (the parts are the waves of
//                          its chunk tiles)
//   [first_chunk, +nu*nc)  chunk tiles: the chains in groups of chain_group, one group after
//                          the other, chunk-major inside a group (so only one group's state
//                          slots need to stay in the L2 at a time)
// Workgroups are persistent: each reads the id of the XCD it runs on, takes tickets from that
// partition's queue until it is empty, then leaves.  So every hand-off of a partition stays in
// one L2 (see the coherence notes in ssd_device.h).  A chunk tile waits only on work with
// smaller tickets of its own queue (its cumsum and bmm tiles and the previous chunk's tile of
// its chains, or its chain's relay item), claimed by workgroups that are running, so every
// wait ends.  A relay item waits on chunk tiles with larger tickets, which other workgroups
// must claim while it runs: so the relay items of a partition run only when the workgroups
// that joined the partition leave room for them (relay_fits, decided once per partition by the
// first relay ticket and read by every chunk tile); otherwise they leave at once and the chunk
// tiles pass the state themselves, in place in the chain's final-state slot.
struct FusedPart {
    int u0, nu, p0, np, pb;
    uint32_t n_cs, first_chunk, n_total;
};

__device__ inline FusedPart fused_part(const SsdArgs& a, int x) {
    FusedPart f;
    f.u0 = a.part_u0[x];
    f.nu = a.part_u0[x + 1] - f.u0;
    f.p0 = f.u0 / a.tpg;
    f.np = f.nu > 0 ? (f.u0 + f.nu - 1) / a.tpg - f.p0 + 1 : 0;
    f.pb = a.part_pb[x];
    f.n_cs = (uint32_t)f.np * a.nchunks;
    f.first_chunk = 2 * f.n_cs + (uint32_t)a.relay * f.nu;
    // block form with the norm in the launch: a norm item per chunk tile, interleaved (norm_ticket)
    f.n_total = f.first_chunk + (uint32_t)f.nu * a.nchunks * (a.norm_fused ? 2u : 1u);
    return f;
}

// Block form with the norm in the launch: the norm items follow all of the partition's chunk
// tiles, in the same chunk-major order, so a norm item waits only on chunk tiles with smaller
// tickets that have (almost always) finished.  Returns, for ticket t >= first_chunk, the chunk
// tile ticket it stands for (first_chunk + c * nu + k), with *norm set for a norm item.
// (Interleaving the norm items a chunk behind the tiles was measured slower: norm items claimed
// while their chunk's tiles still ran held workgroups waiting.)
__device__ inline uint32_t norm_ticket(const FusedPart& f, int nc, uint32_t t, bool* norm) {
    const uint32_t tiles = (uint32_t)f.nu * (uint32_t)nc;
    *norm = t - f.first_chunk >= tiles;
    return *norm ? t - tiles : t;
}

// hardware id of the XCD this wave runs on (HW_REG_XCC_ID, bits [3:0])
__device__ inline uint32_t xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20); }

// The argument block seen through an offset the compiler cannot fold: reading it again on
// every trip of the work loop costs a few scalar loads, while letting the compiler hoist the
// tile code's many argument loads out of the loop keeps them live across the whole tile and
// spills registers.
__device__ inline const SsdArgs& fresh_args(const SsdArgs& a) {
    int zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    return *(const SsdArgs*)((const char*)&a + zero);
}

// The chain and chunk of chunk ticket t (t >= first_chunk of partition f): the chains are taken
// in groups of chain_group, one group after the other, chunk-major inside a group.
struct ChunkItem {
    int b, c, g, tig;
    size_t slot;  // cs_done / bmm_done / cb slot of (pair, c)
};
__device__ inline ChunkItem chunk_item(const SsdArgs& a, const FusedPart& f, uint32_t t) {
    const int nc = a.nchunks, Gn = a.ngroups, tpg = a.tpg;
    const uint32_t v = t - f.first_chunk;
    const int cg = a.chain_group < f.nu ? a.chain_group : f.nu;
    const uint32_t per_group = (uint32_t)cg * nc;
    const int grp = v / per_group;
    const uint32_t w = v - grp * per_group;
    const int gu0 = grp * cg;
    const int gsz = f.nu - gu0 < cg ? f.nu - gu0 : cg;
    const int u = f.u0 + gu0 + (int)(w % gsz);
    const int pair = u / tpg;
    ChunkItem it;
    it.c = w / gsz;
    it.tig = u % tpg;
    it.b = pair / Gn;
    it.g = pair % Gn;
    it.slot = (size_t)(f.pb + pair - f.p0) * nc + it.c;
    return it;
}

// Ticket claimed ahead in the fused form: a chunk tile calls claim() once its round-2 reads
// are issued, so thread 0's atomic on the partition's ticket overlaps the state hop.  The next
// ticket is larger than the current one and runs only after it, so the claim order keeps every
// wait finite.  (Touching the next tile's x rows into the L2 from here was measured slower once
// y left in whole lines: the touched lines pushed state slots out of the L2.)
struct ClaimHook {
    const SsdArgs& a;
    int part;
    uint32_t* s_next;  // LDS
    bool live;         // the partition's relay items run
    __device__ inline void claim() const {
        if (threadIdx.x == 0) *s_next = atomicAdd(a.ticket + part * kTicketStride, 1u);
    }
    __device__ inline bool relay_live() const { return live; }
};

// chunk(args, b, c, g, tig, cb, hook) runs one chunk tile after its cumsum and bmm tiles are done.
// BLK: the block form -- each bmm tile first convolves its chunk's B and C rows (conv_bc_tile);
// BQ: its chunk size (for the norm items).
template <int HPT, int P, typename T, int N, int VL, int BLK = 0, int BQ = 0, typename ChunkFn>
__device__ void fused_loop(const SsdArgs& a0, ChunkFn&& chunk) {
    __shared__ uint32_t s_word, s_next;
    const uint32_t raw = xcc_id();
    const int x = (int)(raw % (uint32_t)a0.nparts);
    const SsdArgs& a = a0;
    // The first workgroup to reach partition x records its XCD; a workgroup from another XCD
    // whose id maps to the same partition leaves it alone (its hand-offs would cross L2s).
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicCAS(a.owner + x, 0u, raw + 1);
        s_word = (prev == 0u || prev == raw + 1) ? 1u : 0u;
        if (s_word) atomicAdd(a.joined + x, 1u);
    }
    __syncthreads();
    const bool mine = __builtin_amdgcn_readfirstlane(s_word) != 0u;
    uint32_t pending = 0xffffffffu;  // a ticket the previous chunk tile claimed ahead
    int live = -1;                   // relay form: the partition's decision, once read
    while (mine) {
        lds_barrier();  // the previous tile is done with LDS and s_word (its stores may still fly)
        const SsdArgs& a = fresh_args(a0);
        uint32_t t = pending;
        if (t == 0xffffffffu) {
            if (threadIdx.x == 0) s_word = atomicAdd(a.ticket + x * kTicketStride, 1u);
            lds_barrier();
            t = __builtin_amdgcn_readfirstlane(s_word);
        }
        pending = 0xffffffffu;
        const FusedPart f = fused_part(a, x);
        const int nc = a.nchunks, Gn = a.ngroups, tpg = a.tpg, hpg = a.hpg, Q = a.chunk;
        if (t >= f.n_total) break;
        if (t < 2 * f.n_cs) {
            const uint32_t v = t < f.n_cs ? t : t - f.n_cs;
            const int c = v / f.np, lp = v % f.np;
            const int pair = f.p0 + lp, b = pair / Gn, g = pair % Gn;
            const size_t slot = (size_t)(f.pb + lp) * nc + c;
            if (t < f.n_cs) {
                // heads of this pair that belong to the partition's chains
                const int lo = (f.u0 > pair * tpg ? f.u0 - pair * tpg : 0) * HPT;
                const int hi_u = f.u0 + f.nu < (pair + 1) * tpg ? f.u0 + f.nu - pair * tpg : tpg;
                const int hi = hi_u * HPT < hpg ? hi_u * HPT : hpg;
                cumsum_tile<T>(a, b, c, g * hpg + lo, g * hpg + hi);
                publish_flag_block(a.cs_done + slot);
            } else {
                if constexpr (BLK) {
                    conv_bc_tile<T, N>(a, b, c, g);
                    wait_vm_all();  // this workgroup's convolved rows are in the L2
                    __syncthreads();
                }
                bmm_tile<T, N>(a, b, c, g, cb_at(a, slot));
                publish_flag_block(a.bmm_done + slot);
            }
        } else if (t < f.first_chunk) {
            // The first relay ticket decides for the partition whether its relay items run: only
            // when the workgroups that joined it (all launched workgroups that found room on the
            // XCD by now; later ones may be waiting for a relay item to end) leave room for them.
            if (threadIdx.x == 0) {
                uint32_t d = __hip_atomic_load(a.relay_on + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (d == 0u) {
                    const int j = (int)__hip_atomic_load(a.joined + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const uint32_t want = (a.relay_admit && relay_fits(a.relay, f.nu, j)) ? 1u : 2u;
                    const uint32_t prev = atomicCAS(a.relay_on + x, 0u, want);
                    d = prev == 0u ? want : prev;
                }
                s_word = d;
            }
            lds_barrier();
            if (__builtin_amdgcn_readfirstlane(s_word) != 1u) continue;  // the chunk tiles hop
            // relay item k of chain u (its chunk tiles' 4 waves are 4 parts, (head hs, p-slice ph)):
            // parts k * PPI .. k * PPI + PPI - 1, R = a.relay waves each
            constexpr int PW = P < 32 ? P : 32, WPH = P / PW, NT = (N / 16) * (PW / 16);
            const int R = a.relay, PPI = 4 / R;
            const uint32_t r = t - 2 * f.n_cs;
            const int wave = __builtin_amdgcn_readfirstlane(tid_here() >> 6), rw = wave % R;
            const int u = f.u0 + (int)(r / R), part = (int)(r % R) * PPI + wave / R;
            const int pair = u / tpg, tig = u % tpg, hs = part / WPH, ph = part % WPH;
            const int b = pair / Gn, h = (pair % Gn) * hpg + tig * HPT + hs;
            if (tig * HPT + hs < hpg && rw < relay_waves_of<T, NT>(a)) {
                if (R == 4)
                    relay_chain<T, NT, 4, VL>(a, b, h, ph, WPH, rw);
                else
                    relay_chain<T, NT, 2, VL>(a, b, h, ph, WPH, rw);
            }
        } else {
            if constexpr (BLK) {
                if (a.norm_fused) {
                    bool norm;
                    t = norm_ticket(f, nc, t, &norm);
                    if (norm) {
                        const ChunkItem it = chunk_item(a, f, t);
                        norm_item<T, P, HPT, BQ>(a, it.b, it.c, it.g, it.tig);
                        continue;
                    }
                }
            }
            const ChunkItem it = chunk_item(a, f, t);
            if (a.relay && live < 0) {
                // the partition's relay decision (made by its first relay ticket, which is smaller)
                if (tid_here() < 64) {
                    wait_flag(a.relay_on + x, a, 1u);
                    if (tid_here() == 0)
                        s_word = __hip_atomic_load(a.relay_on + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                lds_barrier();
                live = __builtin_amdgcn_readfirstlane(s_word) == 1u ? 1 : 0;
            }
            if (tid_here() < 64)  // wave 0: both flags with one poll
                wait_pair(a.cs_done, (uint32_t)it.slot, (uint32_t)(a.bmm_done - a.cs_done + it.slot), a);
            lds_barrier();  // every wave starts after the flags were seen
            const ClaimHook hook{a, x, &s_next, live == 1};
            chunk(a, it.b, it.c, it.g, it.tig, cb_at(a, it.slot), hook);
            lds_barrier();  // s_next holds the ticket claimed ahead
            pending = __builtin_amdgcn_readfirstlane(s_next);
        }
    }
    // The last workgroup to leave checks that every partition's queue was emptied (a
    // partition no workgroup served would leave its outputs unwritten).
    __syncthreads();
    if (threadIdx.x == 0 && atomicAdd(a.exit_count, 1u) == gridDim.x - 1) {
        for (int y = 0; y < a.nparts; ++y) {
            const uint32_t claimed = __hip_atomic_load(a.ticket + y * kTicketStride, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            if (claimed < fused_part(a, y).n_total)
                __hip_atomic_store(a.status, 9u /* SSD_ERR_SCHEDULE */, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <typename T, int P, int N, int VL> __global__ __launch_bounds__(256) void k_fused(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo<T, P, N>::SMEM];
    fused_loop<Geo<T, P, N>::HPT, P, T, N, VL>(a, [&](const SsdArgs& ai, int b, int c, int g, int tig,
                                                      const float* cbp, const auto& hook) {
        hook.claim();
        chunk_tile<T, P, N, MODE_FUSED, VL>(ai, b, c, g, tig, smem, cbp, hook.relay_live());
    });
}

template <typename T, int P, int N, int Q, int VL>
__global__ __launch_bounds__(256, (Geo16<T, P, N, Q>::OCC)) void k_fused16(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo16<T, P, N, Q>::SMEM];
    fused_loop<Geo16<T, P, N, Q>::HPT, P, T, N, VL>(a, [&](const SsdArgs& ai, int b, int c, int g, int tig,
                                                           const float* cbp, const auto& hook) {
        chunk_tile16<T, P, N, Q, MODE_FUSED, VL>(ai, b, c, g, tig, smem, cbp, hook);
    });
}

// The block form: the convolution before and (a.norm_fused) the norm after the SSD in the same
// launch ("Mamba-2炸裂升级！…", section "未来展望与应用拓展").
template <typename T, int P, int N, int Q>
__global__ __launch_bounds__(256, (Geo16<T, P, N, Q>::OCC)) void k_fused16_blk(SsdArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[Geo16<T, P, N, Q>::SMEM];
    fused_loop<Geo16<T, P, N, Q>::HPT, P, T, N, 0, 1, Q>(a, [&](const SsdArgs& ai, int b, int c, int g, int tig,
                                                             const float* cbp, const auto& hook) {
        chunk_tile16<T, P, N, Q, MODE_FUSED, 0, 1>(ai, b, c, g, tig, smem, cbp, hook);
    });
}

// ---- host launchers ----------------------------------------------------------------------
inline hipError_t launch(const void* fn, unsigned grid, void* arg0, hipStream_t st) {
    void* args[] = {arg0};
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, st);
}

// Persistent fused launch: as many workgroups per partition as fit on its XCD at once (and no
// more than its queue holds).  Workgroups are dealt to XCDs round robin, so partition x's
// share arrives on one XCD; fused_loop does not rely on that for correctness.
inline hipError_t fused_occupancy(const void* fn, SsdArgs& a) {
    int occ = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, 256, 0);
    a.fused_occ = occ < 1 ? 1 : occ;
    return e;
}

inline hipError_t launch_fused(const void* fn, SsdArgs& a, hipStream_t st) {
    if (a.fused_occ < 1) {
        const hipError_t e = fused_occupancy(fn, a);
        if (e != hipSuccess) return e;
    }
    const int per_xcd = (a.cu_count / a.nparts > 0 ? a.cu_count / a.nparts : 1) * a.fused_occ;
    const int wgs = per_xcd < a.part_max_work ? per_xcd : a.part_max_work;
    // no group chosen on the host (set_partitions picks one only for many short chains): all of
    // a partition's chains in one group (smaller groups keep fewer state slots live, but long
    // chains then serialise on the chunk-to-chunk hand-off)
    if (a.chain_group <= 0) a.chain_group = 1 << 30;
    unsigned grid = (unsigned)(a.nparts * (wgs > 0 ? wgs : 1));
    const char* lim = getenv("MAMBA_SSD_GRID_LIMIT");  // test knob (see ssd_api.cpp)
    if (lim && *lim && atoi(lim) > 0 && (unsigned)atoi(lim) < grid) grid = (unsigned)atoi(lim);
    return launch(fn, grid, &a, st);
}

// VL: 0 plain input, 1 packed input, 2 packed input with per-sequence states.
template <typename T, int P, int N, int VL> hipError_t launch_step_t(int step, SsdArgs& a, hipStream_t st) {
    typedef Geo<T, P, N> G_;
    const unsigned Bn = a.batch, nc = a.nchunks, Gn = a.ngroups, tpg = a.tpg;
    switch (step) {
    case STEP_CUMSUM:
        return launch((const void*)&k_chunk_cumsum<T>, Bn * nc, &a, st);
    case STEP_BMM:
        return launch((const void*)&k_bmm<T, N>, Bn * nc * Gn, &a, st);
    case STEP_CHUNK_STATE:
        return launch((const void*)&k_chunk<T, P, N, MODE_STATE, VL>, Bn * nc * Gn * tpg, &a, st);
    case STEP_STATE_PASSING:
        return launch_state_passing(a, P * N, st);
    case STEP_CHUNK_SCAN:
        return launch((const void*)&k_chunk<T, P, N, MODE_SCAN, VL>, Bn * nc * Gn * tpg, &a, st);
    case STEP_FUSED:
        return launch_fused((const void*)&k_fused<T, P, N, VL>, a, st);
    case STEP_FUSED_OCCUPANCY:
        return fused_occupancy((const void*)&k_fused<T, P, N, VL>, a);
    default:
        return hipErrorInvalidValue;
    }
    (void)sizeof(G_);
}

template <typename T, int P, int N, int Q, int VL> hipError_t launch_step16(int step, SsdArgs& a, hipStream_t st) {
    const unsigned Bn = a.batch, nc = a.nchunks, Gn = a.ngroups, tpg = a.tpg;
    switch (step) {
    case STEP_CUMSUM:
        return launch((const void*)&k_chunk_cumsum<T>, Bn * nc, &a, st);
    case STEP_BMM:
        return launch((const void*)&k_bmm<T, N>, Bn * nc * Gn, &a, st);
    case STEP_CHUNK_STATE:
        return launch((const void*)&k_chunk16<T, P, N, Q, MODE_STATE, VL>, Bn * nc * Gn * tpg, &a, st);
    case STEP_STATE_PASSING:
        return launch_state_passing(a, P * N, st);
    case STEP_CHUNK_SCAN:
        return launch((const void*)&k_chunk16<T, P, N, Q, MODE_SCAN, VL>, Bn * nc * Gn * tpg, &a, st);
    case STEP_FUSED:
        return launch_fused((const void*)&k_fused16<T, P, N, Q, VL>, a, st);
    case STEP_FUSED_OCCUPANCY:
        return fused_occupancy((const void*)&k_fused16<T, P, N, Q, VL>, a);
    default:
        return hipErrorInvalidValue;
    }
}

// The (headdim, dstate) pairs each input type supports, dispatched to launch_step16 /
// launch_step_t; hipErrorNotSupported otherwise.  One translation unit instantiates one
// (type, chunk size, VL) combination.
template <typename T, int Q, int VL> hipError_t dispatch16(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    if (P == 16 && N == 32) return launch_step16<T, 16, 32, Q, VL>(step, a, st);
    if (P == 16 && N == 64) return launch_step16<T, 16, 64, Q, VL>(step, a, st);
    if (P == 16 && N == 128) return launch_step16<T, 16, 128, Q, VL>(step, a, st);
    if (P == 32 && N == 32) return launch_step16<T, 32, 32, Q, VL>(step, a, st);
    if (P == 32 && N == 64) return launch_step16<T, 32, 64, Q, VL>(step, a, st);
    if (P == 32 && N == 128) return launch_step16<T, 32, 128, Q, VL>(step, a, st);
    if (P == 64 && N == 32) return launch_step16<T, 64, 32, Q, VL>(step, a, st);
    if (P == 64 && N == 64) return launch_step16<T, 64, 64, Q, VL>(step, a, st);
    if (P == 64 && N == 128) return launch_step16<T, 64, 128, Q, VL>(step, a, st);
    if (P == 128 && N == 32) return launch_step16<T, 128, 32, Q, VL>(step, a, st);
    if (P == 128 && N == 64) return launch_step16<T, 128, 64, Q, VL>(step, a, st);
    if (P == 128 && N == 128) return launch_step16<T, 128, 128, Q, VL>(step, a, st);
    return hipErrorNotSupported;
}

// The block form's (headdim, dstate) pairs: P in {64, 128} (whole token rows of y in LDS for
// the norm), N in {64, 128}.
template <typename T, int Q> hipError_t dispatch_blk16(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    const void* fn = nullptr;
    if (P == 64 && N == 64) fn = (const void*)&k_fused16_blk<T, 64, 64, Q>;
    else if (P == 64 && N == 128) fn = (const void*)&k_fused16_blk<T, 64, 128, Q>;
    else if (P == 128 && N == 64) fn = (const void*)&k_fused16_blk<T, 128, 64, Q>;
    else if (P == 128 && N == 128) fn = (const void*)&k_fused16_blk<T, 128, 128, Q>;
    else return hipErrorNotSupported;
    if (step == STEP_FUSED) return launch_fused(fn, a, st);
    if (step == STEP_FUSED_OCCUPANCY) return fused_occupancy(fn, a);
    return hipErrorInvalidValue;
}

template <int VL> hipError_t dispatch32(int step, int P, int N, SsdArgs& a, hipStream_t st) {
    if (P == 16 && N == 16) return launch_step_t<float, 16, 16, VL>(step, a, st);
    if (P == 16 && N == 32) return launch_step_t<float, 16, 32, VL>(step, a, st);
    if (P == 16 && N == 64) return launch_step_t<float, 16, 64, VL>(step, a, st);
    if (P == 16 && N == 128) return launch_step_t<float, 16, 128, VL>(step, a, st);
    if (P == 32 && N == 16) return launch_step_t<float, 32, 16, VL>(step, a, st);
    if (P == 32 && N == 32) return launch_step_t<float, 32, 32, VL>(step, a, st);
    if (P == 32 && N == 64) return launch_step_t<float, 32, 64, VL>(step, a, st);
    if (P == 32 && N == 128) return launch_step_t<float, 32, 128, VL>(step, a, st);
    if (P == 64 && N == 16) return launch_step_t<float, 64, 16, VL>(step, a, st);
    if (P == 64 && N == 32) return launch_step_t<float, 64, 32, VL>(step, a, st);
    if (P == 64 && N == 64) return launch_step_t<float, 64, 64, VL>(step, a, st);
    if (P == 64 && N == 128) return launch_step_t<float, 64, 128, VL>(step, a, st);
    if (P == 128 && N == 16) return launch_step_t<float, 128, 16, VL>(step, a, st);
    if (P == 128 && N == 32) return launch_step_t<float, 128, 32, VL>(step, a, st);
    if (P == 128 && N == 64) return launch_step_t<float, 128, 64, VL>(step, a, st);
    if (P == 128 && N == 128) return launch_step_t<float, 128, 128, VL>(step, a, st);
    return hipErrorNotSupported;
}

}  // namespace ssd
