// ssd_api.cpp -- the C ABI declared in include/mamba_ssd.h: argument validation (host
// only, before any HIP call), workspace carve-up and kernel dispatch.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/mamba_ssd.h"
#include "ssd_api_internal.h"
#include "ssd_launch.h"

#define SSD_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kAlign = 256;       // workspace region alignment
// Fused form: shapes with at most this many chains (b, g, tile-in-group) get the relay form's
// buffers and use it when every partition has enough workgroups (see set_partitions).
constexpr int64_t kRelayMaxChains = 128;
constexpr uint32_t kDefaultSpin = 1u << 22;

size_t elem_size(int dt) { return dt == SSD_F32 ? 4 : 2; }

// ssd_params_t of ABI version 1 ended before `relaxed`; such callers get relaxed = 0.
constexpr size_t kParamsV1Size = offsetof(ssd_params_t, relaxed);
int relaxed(const ssd_params_t* p) { return p->struct_size >= sizeof(ssd_params_t) ? p->relaxed : 0; }
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// MAMBA_SSD_SPIN_LIMIT: polls after which a fused-kernel wait gives up (read on every call, so
// a test can make the kernel's own bounded waits give up and then run normally again).
uint32_t spin_limit() {
    const char* e = getenv("MAMBA_SSD_SPIN_LIMIT");
    if (!e || !*e) return kDefaultSpin;
    const unsigned long x = strtoul(e, nullptr, 10);
    return x ? (uint32_t)(x > 0xffffffffUL ? 0xffffffffUL : x) : kDefaultSpin;
}

// Test knobs of the fused form, read on every call: MAMBA_SSD_RELAY_ADMIT=0 makes every
// partition of a relay-form launch decide that its chunk tiles pass the state themselves;
// MAMBA_SSD_GRID_LIMIT=n caps the fused grid at n workgroups (partitions left without a
// workgroup are then reported as SSD_ERR_SCHEDULE).
int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    if (!e || !*e) return dflt;
    return (int)strtol(e, nullptr, 10);
}

// MAMBA_SSD_CHAIN_GROUP: chains per claim group of the fused kernel (unset or 0: automatic,
// see set_partitions).  Read on every call.
int chain_group_env() {
    const char* e = getenv("MAMBA_SSD_CHAIN_GROUP");
    if (!e || !*e) return 0;
    const long x = strtol(e, nullptr, 10);
    return x > 0 && x < (1L << 30) ? (int)x : 0;
}

// MAMBA_SSD_RELAY: "0" never uses the fused relay form; "1" uses it whenever a partition has
// enough workgroups, "2" / "4" also fix its relay waves per chain part; unset: by shape
// (kRelayMaxChains).  Read on every call.
int relay_env() {
    const char* e = getenv("MAMBA_SSD_RELAY");
    if (!e || !*e) return -1;
    return e[0] == '0' ? 0 : (e[0] == '2' ? 2 : (e[0] == '4' ? 4 : 1));
}

int64_t chain_count(const ssd_params_t* p) {
    const int64_t hpg = p->nheads / p->ngroups, hpt = ssd::heads_per_tile(p->headdim);
    return (int64_t)p->batch * p->ngroups * ((hpg + hpt - 1) / hpt);
}

// Whether the workspace carries the relay form's buffers (fused form only).
bool relay_capable(const ssd_params_t* p) {
    if (p->impl != SSD_IMPL_FUSED) return false;
    const int env = relay_env();
    return env >= 0 ? env != 0 : chain_count(p) <= kRelayMaxChains;
}

// Relaxed intermediates with 16-bit inputs: CB (C B^T of each chunk) stored in the input type.
bool cb16(const ssd_params_t* p) { return relaxed(p) && p->in_dtype != SSD_F32; }

// Relay form with fp16 state storage (16-bit inputs): the chunk states handed to the relay
// items are stored as fp16 too, like every other inter-chunk state of that storage mode.
bool agg16(const ssd_params_t* p) { return p->state_dtype == SSD_F16 && p->in_dtype != SSD_F32; }

struct Layout {
    ssd_workspace_layout_t w;
    // sync words: [flags | cs_done | bmm_done | tickets | owners | exit | abort | status]
    size_t nflags, nsync;
    size_t flags_w, cs_w, bmm_w, ticket_w, owner_w, exit_w, abort_w, status_w;
    size_t agg_bytes;  // relay form: bytes of the chunk-state ring at the start of `s`
    int tpg, wph, op_slots, agg_slots;
};

// Upper bound of the fused form's (b, g) pair slots: the B*G pairs, plus one more for every
// partition boundary that splits a pair (each side keeps its own cumsum / bmm copy).
size_t pair_slots_max(const ssd_params_t* p) { return (size_t)p->batch * p->ngroups + ssd::kMaxXcc - 1; }

ssd_status_t validate(const ssd_params_t* p) {
    if (!p) return SSD_ERR_NULL_POINTER;
    if (p->struct_size < kParamsV1Size) return SSD_ERR_INVALID_ARGUMENT;
    if (p->struct_size >= sizeof(ssd_params_t) &&
        ((p->relaxed != 0 && p->relaxed != 1) || (p->flags & ~SSD_FLAG_WORKSPACE_READY) != 0))
        return SSD_ERR_INVALID_ARGUMENT;
    if (p->in_dtype < SSD_F32 || p->in_dtype > SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
    if (p->state_dtype < SSD_F32 || p->state_dtype > SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
    if (p->impl != SSD_IMPL_UNFUSED && p->impl != SSD_IMPL_FUSED) return SSD_ERR_INVALID_ARGUMENT;
    if (p->dt_softplus != 0 && p->dt_softplus != 1) return SSD_ERR_INVALID_ARGUMENT;
    if (p->batch < 1 || p->seqlen < 1 || p->nheads < 1 || p->headdim < 1 || p->dstate < 1 || p->ngroups < 1 ||
        p->chunk_size < 1)
        return SSD_ERR_INVALID_SHAPE;
    if (p->nheads % p->ngroups) return SSD_ERR_INVALID_SHAPE;
    const int P = p->headdim, N = p->dstate, Q = p->chunk_size;
    if (P != 16 && P != 32 && P != 64 && P != 128) return SSD_ERR_UNSUPPORTED;
    if (N != 32 && N != 64 && N != 128 && !(N == 16 && p->in_dtype == SSD_F32)) return SSD_ERR_UNSUPPORTED;
    if (Q != 64 && Q != 128 && Q != 256) return SSD_ERR_UNSUPPORTED;
    // every grid and ticket count must fit a signed 32-bit index
    const int64_t nc = ((int64_t)p->seqlen + Q - 1) / Q;
    const int64_t hpg = p->nheads / p->ngroups;
    const int64_t tpg = (hpg + ssd::heads_per_tile(P) - 1) / ssd::heads_per_tile(P);
    const int64_t pairs = (int64_t)p->batch * p->ngroups;
    const int64_t tickets = nc * (2 * (pairs + ssd::kMaxXcc) + pairs * tpg) + 4 * pairs * tpg;
    if (tickets >= (int64_t)1 << 31) return SSD_ERR_INVALID_SHAPE;
    if ((int64_t)p->batch * p->seqlen * p->nheads >= (int64_t)1 << 40) return SSD_ERR_INVALID_SHAPE;
    return SSD_OK;
}

Layout layout(const ssd_params_t* p) {
    Layout l{};
    const size_t B = p->batch, L = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate, G = p->ngroups;
    const size_t Q = p->chunk_size, nc = (L + Q - 1) / Q;
    const bool fused = p->impl == SSD_IMPL_FUSED;
    l.wph = ssd::waves_per_head(p->headdim);
    const int hpt = ssd::heads_per_tile(p->headdim);
    l.tpg = (int)((H / G + hpt - 1) / hpt);
    // fused: one state slot per chain, updated in place; relay form: the initial and the final
    // state (the states in between go through its operand ring)
    const bool relay = relay_capable(p);
    const size_t K = fused ? (relay ? 2 : 1) : nc + 1;
    ssd_workspace_layout_t& w = l.w;
    w.nchunks = (int)nc;
    w.state_slots = (int)K;
    w.dt_bytes = B * nc * H * Q * 4;
    w.acs_bytes = w.dt_bytes;
    const size_t PS = fused ? pair_slots_max(p) : 0;
    w.cb_bytes = (fused ? PS : B * G) * nc * Q * Q * (cb16(p) ? 2 : 4);
    // relay form: the chunk-state ring (fp32) and then the operand ring (input dtype)
    l.op_slots = (int)(nc + 1 < (size_t)ssd::kRelaySlots ? nc + 1 : (size_t)ssd::kRelaySlots);
    l.agg_slots = nc > (size_t)ssd::kLongChainChunks ? ssd::kAggSlotsLong : ssd::kAggSlots;
    l.agg_bytes = B * H * P * N * (agg16(p) ? 2 : 4) * (size_t)l.agg_slots;
    w.s_bytes = fused ? (relay ? l.agg_bytes + B * H * P * N * elem_size(p->in_dtype) * l.op_slots : 0)
                      : B * nc * H * P * N * 4;
    w.states_bytes = B * K * H * P * N * elem_size(p->state_dtype);
    w.seg_bytes = B * nc * Q * 4;
    l.nflags = fused ? B * H * (size_t)l.wph * ssd::kChainStride : 0;
    l.flags_w = 0;
    l.cs_w = l.nflags;
    l.bmm_w = l.cs_w + PS * nc;
    l.ticket_w = l.bmm_w + PS * nc;
    l.owner_w = l.ticket_w + (fused ? (size_t)ssd::kMaxXcc * ssd::kTicketStride : 0);
    l.exit_w = l.owner_w + (fused ? 3 * ssd::kMaxXcc : 0);  // owner, joined, relay_on words
    l.abort_w = l.exit_w + (fused ? 1 : 0);
    l.status_w = l.abort_w + 1;
    l.nsync = l.status_w + 1;
    w.sync_bytes = l.nsync * 4;
    size_t off = 0;
    w.dt_offset = off;
    off = align_up(off + w.dt_bytes);
    w.acs_offset = off;
    off = align_up(off + w.acs_bytes);
    w.cb_offset = off;
    off = align_up(off + w.cb_bytes);
    w.s_offset = off;
    off = align_up(off + w.s_bytes);
    w.states_offset = off;
    off = align_up(off + w.states_bytes);
    w.seg_offset = off;
    off = align_up(off + w.seg_bytes);
    w.sync_offset = off;
    w.status_offset = off + 4 * l.status_w;
    off = align_up(off + w.sync_bytes);
    w.total_bytes = off;
    return l;
}

ssd_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return SSD_OK;
    if (e == hipErrorNotSupported) return SSD_ERR_UNSUPPORTED;
    return SSD_ERR_HIP;
}

hipError_t dispatch(int step, const ssd_params_t* p, ssd::SsdArgs& a, hipStream_t st) {
    switch (p->in_dtype) {
    case SSD_F32: return ssd::launch_step_f32(step, p->headdim, p->dstate, a, st);
    case SSD_F16: return ssd::launch_step_f16(step, p->headdim, p->dstate, a, st);
    default: return ssd::launch_step_bf16(step, p->headdim, p->dstate, a, st);
    }
}

// Kernel argument block with every workspace pointer filled in; tensor pointers are set
// by the callers.
ssd::SsdArgs make_args(const ssd_params_t* p, const Layout& l, void* ws) {
    ssd::SsdArgs a{};
    char* base = (char*)ws;
    a.dtf = (float*)(base + l.w.dt_offset);
    a.acs = (float*)(base + l.w.acs_offset);
    a.cb = (float*)(base + l.w.cb_offset);
    a.s = (float*)(base + l.w.s_offset);
    a.opnd = base + l.w.s_offset + l.agg_bytes;
    a.op_slots = l.op_slots;
    a.states = base + l.w.states_offset;
    a.seg = (int*)(base + l.w.seg_offset);
    uint32_t* sync = (uint32_t*)(base + l.w.sync_offset);
    a.flags = sync + l.flags_w;
    a.cs_done = sync + l.cs_w;
    a.bmm_done = sync + l.bmm_w;
    a.ticket = sync + l.ticket_w;
    a.owner = sync + l.owner_w;
    a.joined = a.owner + ssd::kMaxXcc;
    a.relay_on = a.owner + 2 * ssd::kMaxXcc;
    a.exit_count = sync + l.exit_w;
    a.abort_word = sync + l.abort_w;
    a.status = sync + l.status_w;
    a.batch = p->batch;
    a.seqlen = p->seqlen;
    a.nheads = p->nheads;
    a.ngroups = p->ngroups;
    a.chunk = p->chunk_size;
    a.nchunks = l.w.nchunks;
    a.hpg = p->nheads / p->ngroups;
    a.tpg = l.tpg;
    a.slots = l.w.state_slots;
    a.state_dtype = p->state_dtype;
    a.softplus = p->dt_softplus;
    a.agg16 = agg16(p);
    a.agg_slots = l.agg_slots;
    a.cb16 = cb16(p);
    a.spin_limit = spin_limit();
    a.x_stride = p->nheads * p->headdim;
    return a;
}

// Per-device facts the fused launch needs: its XCD count (the number of work partitions,
// at most kMaxXcc) and compute-unit count.
struct DevInfo {
    int nparts, cus;
};

hipError_t device_info(DevInfo* out) {
    static std::mutex mu;
    static DevInfo cache[64];
    static bool have[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < 64 && have[dev]) {
        *out = cache[dev];
        return hipSuccess;
    }
    int xcc = 1, cus = 1;
    e = hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    DevInfo d;
    d.nparts = xcc < 1 ? 1 : (xcc > ssd::kMaxXcc ? ssd::kMaxXcc : xcc);
    d.cus = cus < 1 ? 1 : cus;
    if (dev >= 0 && dev < 64) {
        cache[dev] = d;
        have[dev] = true;
    }
    *out = d;
    return hipSuccess;
}

constexpr int64_t kL2Bytes = 4 << 20;  // L2 per XCD on MI355X
constexpr int64_t kShortChain = 8;      // chunks per chain up to which the chains are claimed in groups

// Fused form: split the U = B*G*tpg chains into nparts contiguous, near-equal ranges and give
// each partition's (b, g) pairs consecutive cb / flag slots.
void set_partitions(const ssd_params_t* p, const Layout& l, const DevInfo& d, ssd::SsdArgs& a) {
    const int64_t U = (int64_t)p->batch * p->ngroups * l.tpg;
    const int64_t nc = l.w.nchunks;
    a.nparts = d.nparts;
    a.cu_count = d.cus;
    a.chain_group = chain_group_env();
    a.relay_admit = env_int("MAMBA_SSD_RELAY_ADMIT", 1) != 0;
    int pb = 0, maxw = 0, maxu = 0;
    for (int x = 0; x <= d.nparts; ++x) {
        a.part_u0[x] = (int)(U * x / d.nparts);
        a.part_pb[x] = pb;
        if (x == d.nparts) break;
        const int u0 = (int)(U * x / d.nparts), u1 = (int)(U * (x + 1) / d.nparts);
        const int np = u1 > u0 ? (u1 - 1) / l.tpg - u0 / l.tpg + 1 : 0;
        pb += np;
        const int64_t work = nc * (2 * np + (u1 - u0)) + 4 * (u1 - u0);
        if (work > maxw) maxw = (int)work;
        if (u1 - u0 > maxu) maxu = u1 - u0;
    }
    a.part_max_work = maxw;
    // The relay items (R per chain, R = relay waves per chain part) hold one workgroup each
    // for the whole launch: use them only while they fit (relay_fits) in the workgroups a
    // partition holds at once (its CUs times the fused kernel's real occupancy).  The kernel
    // checks the same rule again against the workgroups that actually joined each partition,
    // and falls back to the chunk tiles' own hop where it fails (see fused_loop).
    // R = 4 halves each relay wave's share of the state (faster hand-offs) and is used while
    // the chunk tiles still have 16 workgroups per chain; else R = 2 (more chunk tiles at once).
    const int per_part = (d.cus / d.nparts > 0 ? d.cus / d.nparts : 1) * (a.fused_occ > 0 ? a.fused_occ : 1);
    auto usable = [&](int R) { return ssd::relay_fits(R, maxu, per_part); };
    const int env = relay_env();
    a.relay = 0;
    if (relay_capable(p)) {
        if (env == 2 || env == 4)
            a.relay = usable(env) ? env : 0;
        else if (per_part - 4 * maxu >= 16 * maxu)
            a.relay = 4;
        else if (usable(2))
            a.relay = 2;
    }
    a.slots = a.relay ? l.w.state_slots : 1;
    // Claim groups (hop form, no MAMBA_SSD_CHAIN_GROUP): claimed chunk-major over all of a
    // partition's chains, every chain's state slot is live at once.  When those slots far exceed
    // the XCD's L2 and the chains are short, claiming the chains in groups whose slots fill half
    // the L2 keeps each hop's state there (measured on MI355X, 32 × 1024-token G8 batch: 8-chunk
    // chains 0.93 -> 0.84 ms, 4-chunk chains 1.77 -> 1.65 ms; 16-chunk chains unchanged).  Long
    // chains stay in one group: in small groups the chunk tiles of a chain run close together
    // and wait on each other's hops (2.7B layer, 64-chunk chains in groups of 32: 0.85 -> 0.99 ms).
    if (a.chain_group == 0 && a.relay == 0 && nc <= kShortChain) {
        const int64_t slot = (int64_t)ssd::heads_per_tile(p->headdim) * p->headdim * p->dstate *
                             (int64_t)elem_size(p->state_dtype);
        if ((int64_t)maxu * slot > 2 * kL2Bytes) a.chain_group = (int)std::max<int64_t>(8, kL2Bytes / 2 / slot);
    }
}

// Workspaces whose synchronisation words the last fused call reset for the next one (in its
// final-state copy), with what that call was: a call flagged SSD_FLAG_WORKSPACE_READY skips
// the reset launch only when it is the same.  A few entries; the oldest is dropped.
struct ReadyKey {
    const void* ws;
    ssd_params_t p;  // flags cleared
    int relay, slots;
    size_t nsync;
    bool operator==(const ReadyKey& o) const {
        return ws == o.ws && memcmp(&p, &o.p, sizeof(p)) == 0 && relay == o.relay && slots == o.slots &&
               nsync == o.nsync;
    }
};
constexpr int kReadyEntries = 16;
std::mutex ready_mu;
ReadyKey ready_tab[kReadyEntries];
int ready_n = 0;

ReadyKey ready_key(const ssd_params_t* p, const void* ws, int relay, int slots, size_t nsync) {
    ReadyKey k;
    memset(&k, 0, sizeof(k));
    k.ws = ws;
    memcpy(&k.p, p, p->struct_size < sizeof(k.p) ? p->struct_size : sizeof(k.p));
    k.p.struct_size = sizeof(k.p);
    k.p.flags = 0;
    if (p->struct_size < sizeof(ssd_params_t)) k.p.relaxed = 0;
    k.relay = relay;
    k.slots = slots;
    k.nsync = nsync;
    return k;
}

// Drops the workspace's entry; returns whether it matched k.
bool ready_take(const ReadyKey& k) {
    std::lock_guard<std::mutex> lock(ready_mu);
    for (int i = 0; i < ready_n; ++i) {
        if (ready_tab[i].ws != k.ws) continue;
        const bool same = ready_tab[i] == k;
        ready_tab[i] = ready_tab[--ready_n];
        return same;
    }
    return false;
}

void ready_drop(const void* ws) {
    std::lock_guard<std::mutex> lock(ready_mu);
    for (int i = 0; i < ready_n; ++i)
        if (ready_tab[i].ws == ws) ready_tab[i] = ready_tab[--ready_n];
}

void ready_put(const ReadyKey& k) {
    std::lock_guard<std::mutex> lock(ready_mu);
    for (int i = 0; i < ready_n; ++i)
        if (ready_tab[i].ws == k.ws) ready_tab[i] = ready_tab[--ready_n];
    if (ready_n == kReadyEntries) {
        for (int i = 1; i < ready_n; ++i) ready_tab[i - 1] = ready_tab[i];
        --ready_n;
    }
    ready_tab[ready_n++] = k;
}

// Validates and lays out; a call that will write the workspace forgets that it was left ready
// (keep_ready: the fused form, which looks the entry up itself).
ssd_status_t check_ws(const ssd_params_t* p, void* ws, size_t ws_bytes, Layout* l, bool keep_ready = false) {
    ssd_status_t s = validate(p);
    if (s != SSD_OK) return s;
    if (!ws) return SSD_ERR_NULL_POINTER;
    if (!aligned(ws, kAlign)) return SSD_ERR_MISALIGNED;
    *l = layout(p);
    if (ws_bytes < l->w.total_bytes) return SSD_ERR_WORKSPACE_TOO_SMALL;
    if (!keep_ready) ready_drop(ws);
    return SSD_OK;
}

size_t state_bytes_per_b(const ssd_params_t* p) {
    return (size_t)p->nheads * p->headdim * p->dstate * elem_size(p->state_dtype);
}

// Boundary copy into slot 0 (initial state or zeros); optionally resets sync words.
hipError_t boundary_in(const ssd_params_t* p, const Layout& l, const ssd::SsdArgs& a, const void* h0,
                       uint32_t* sync, size_t nsync, size_t nflags, hipStream_t st) {
    const size_t per_b = state_bytes_per_b(p);
    return ssd::launch_boundary(h0, per_b, a.states, per_b * l.w.state_slots, per_b, p->batch, sync, nsync, nflags,
                                (uint32_t)(l.w.nchunks + 1), st);
}

hipError_t boundary_out(const ssd_params_t* p, const Layout& l, const ssd::SsdArgs& a, void* fin, hipStream_t st) {
    const size_t per_b = state_bytes_per_b(p);
    const int slot = l.w.nchunks % l.w.state_slots;
    return ssd::launch_boundary((const char*)a.states + per_b * slot, per_b * l.w.state_slots, fin, per_b, per_b,
                                p->batch, nullptr, 0, 0, 1, st);
}

}  // namespace

SSD_EXPORT ssd_status_t ssd_validate(const ssd_params_t* p) { return validate(p); }

SSD_EXPORT size_t ssd_prefill_workspace_size(const ssd_params_t* p) {
    if (validate(p) != SSD_OK) return 0;
    return layout(p).w.total_bytes;
}

SSD_EXPORT ssd_status_t ssd_workspace_layout(const ssd_params_t* p, ssd_workspace_layout_t* out) {
    ssd_status_t s = validate(p);
    if (s != SSD_OK) return s;
    if (!out) return SSD_ERR_NULL_POINTER;
    *out = layout(p).w;
    return SSD_OK;
}

SSD_EXPORT const char* ssd_status_string(ssd_status_t s) {
    switch (s) {
    case SSD_OK: return "success";
    case SSD_ERR_NULL_POINTER: return "a required pointer is NULL";
    case SSD_ERR_INVALID_SHAPE: return "invalid shape (size < 1, nheads % ngroups != 0, or index overflow)";
    case SSD_ERR_UNSUPPORTED: return "unsupported headdim / dstate / chunk_size / dtype combination";
    case SSD_ERR_MISALIGNED: return "a pointer is not aligned as required";
    case SSD_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than ssd_prefill_workspace_size()";
    case SSD_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case SSD_ERR_SYNC_TIMEOUT: return "a cross-workgroup wait hit its spin limit; outputs are invalid";
    case SSD_ERR_INVALID_ARGUMENT: return "an enum field is out of range or struct_size is too small";
    case SSD_ERR_SCHEDULE: return "fused kernel: a work partition was not served by any workgroup; outputs are invalid";
    case SSD_ERR_SCRATCH_TOO_SMALL:
        return "ssd_prefill_noalloc: the problem needs more workspace than the library's static scratch holds";
    default: return "unknown status";
    }
}

// ---- the five unfused steps ---------------------------------------------------------------

static ssd_status_t unfused_guard(const ssd_params_t* p) {
    if (p && p->struct_size >= kParamsV1Size && p->impl != SSD_IMPL_UNFUSED) return SSD_ERR_INVALID_ARGUMENT;
    return SSD_OK;
}

SSD_EXPORT ssd_status_t ssd_step_chunk_cumsum(const ssd_params_t* p, const void* dt, const float* A,
                                              const float* dt_bias, void* workspace, size_t workspace_bytes,
                                              void* stream) {
    Layout l;
    ssd_status_t s = unfused_guard(p);
    if (s == SSD_OK) s = check_ws(p, workspace, workspace_bytes, &l);
    if (s != SSD_OK) return s;
    if (!dt || !A) return SSD_ERR_NULL_POINTER;
    if (!aligned(dt, elem_size(p->in_dtype)) || !aligned(A, 4) || !aligned(dt_bias, 4)) return SSD_ERR_MISALIGNED;
    ssd::SsdArgs a = make_args(p, l, workspace);
    a.dt = dt;
    a.A = A;
    a.dt_bias = dt_bias;
    return hip_status(dispatch(ssd::STEP_CUMSUM, p, a, (hipStream_t)stream));
}

SSD_EXPORT ssd_status_t ssd_step_bmm(const ssd_params_t* p, const void* B, const void* C, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    Layout l;
    ssd_status_t s = unfused_guard(p);
    if (s == SSD_OK) s = check_ws(p, workspace, workspace_bytes, &l);
    if (s != SSD_OK) return s;
    if (!B || !C) return SSD_ERR_NULL_POINTER;
    if (!aligned(B, 16) || !aligned(C, 16)) return SSD_ERR_MISALIGNED;
    ssd::SsdArgs a = make_args(p, l, workspace);
    a.B = B;
    a.C = C;
    return hip_status(dispatch(ssd::STEP_BMM, p, a, (hipStream_t)stream));
}

SSD_EXPORT ssd_status_t ssd_step_chunk_state(const ssd_params_t* p, const void* x, const void* B, void* workspace,
                                             size_t workspace_bytes, void* stream) {
    Layout l;
    ssd_status_t s = unfused_guard(p);
    if (s == SSD_OK) s = check_ws(p, workspace, workspace_bytes, &l);
    if (s != SSD_OK) return s;
    if (!x || !B) return SSD_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(B, 16)) return SSD_ERR_MISALIGNED;
    ssd::SsdArgs a = make_args(p, l, workspace);
    a.x = x;
    a.B = B;
    return hip_status(dispatch(ssd::STEP_CHUNK_STATE, p, a, (hipStream_t)stream));
}

SSD_EXPORT ssd_status_t ssd_step_state_passing(const ssd_params_t* p, const void* initial_state, void* final_state,
                                               void* workspace, size_t workspace_bytes, void* stream) {
    Layout l;
    ssd_status_t s = unfused_guard(p);
    if (s == SSD_OK) s = check_ws(p, workspace, workspace_bytes, &l);
    if (s != SSD_OK) return s;
    if (!final_state) return SSD_ERR_NULL_POINTER;
    if (!aligned(initial_state, 16) || !aligned(final_state, 16)) return SSD_ERR_MISALIGNED;
    ssd::SsdArgs a = make_args(p, l, workspace);
    hipStream_t st = (hipStream_t)stream;
    // initial state into slot 0, and clear the status word (the unfused form never waits)
    hipError_t e = boundary_in(p, l, a, initial_state, a.status, 1, 0, st);
    if (e == hipSuccess) e = ssd::launch_state_passing(a, p->headdim * p->dstate, st);
    if (e == hipSuccess) e = boundary_out(p, l, a, final_state, st);
    return hip_status(e);
}

SSD_EXPORT ssd_status_t ssd_step_chunk_scan(const ssd_params_t* p, const void* x, const void* C, const float* D,
                                            void* y, void* workspace, size_t workspace_bytes, void* stream) {
    Layout l;
    ssd_status_t s = unfused_guard(p);
    if (s == SSD_OK) s = check_ws(p, workspace, workspace_bytes, &l);
    if (s != SSD_OK) return s;
    if (!x || !C || !y) return SSD_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(D, 4)) return SSD_ERR_MISALIGNED;
    ssd::SsdArgs a = make_args(p, l, workspace);
    a.x = x;
    a.C = C;
    a.D = D;
    a.y = y;
    return hip_status(dispatch(ssd::STEP_CHUNK_SCAN, p, a, (hipStream_t)stream));
}

// ---- the whole prefill ----------------------------------------------------------------------

ssd_status_t ssd::prefill_impl(const ssd_params_t* p, const void* x, const void* dt, const float* A, const void* B,
                               const void* C, const float* D, const float* dt_bias, const void* initial_state,
                               void* y, void* final_state, void* workspace, size_t workspace_bytes, void* stream,
                               hipEvent_t ev_begin, hipEvent_t ev_end, const int32_t* seq_idx,
                               const ssd::SeqStates& ss) {
    Layout l;
    ssd_status_t s = check_ws(p, workspace, workspace_bytes, &l, p && p->impl == SSD_IMPL_FUSED);
    if (s != SSD_OK) return s;
    const bool seqst = ss.final_ != nullptr;
    if (seqst && p->in_dtype == SSD_F32) return SSD_ERR_UNSUPPORTED;
    if (!aligned(seq_idx, 4) || !aligned(ss.initial, 16) || !aligned(ss.final_, 16)) return SSD_ERR_MISALIGNED;
    if (!x || !dt || !A || !B || !C || !y || (!final_state && !seqst)) return SSD_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(final_state, 16) ||
        !aligned(initial_state, 16) || !aligned(dt, elem_size(p->in_dtype)) || !aligned(A, 4) || !aligned(D, 4) ||
        !aligned(dt_bias, 4))
        return SSD_ERR_MISALIGNED;
    hipStream_t st = (hipStream_t)stream;
    ssd::SsdArgs a = make_args(p, l, workspace);
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.dt_bias = dt_bias;
    a.seq_idx = seq_idx;
    a.seqstates = seqst ? 1 : 0;
    a.nseq = ss.nseq;
    a.seq_h0 = ss.initial;
    a.seq_fin = ss.final_;
    a.y = y;
    a.has_h0 = initial_state != nullptr;
    hipError_t e;
    auto mark = [&](hipEvent_t ev) { return ev ? hipEventRecord(ev, st) : hipSuccess; };
    if (p->impl == SSD_IMPL_FUSED) {
        DevInfo d;
        e = device_info(&d);
        if (e == hipSuccess) e = dispatch(ssd::STEP_FUSED_OCCUPANCY, p, a, st);
        if (e != hipSuccess) return hip_status(e);
        set_partitions(p, l, d, a);
        if (seqst) {
            // per-sequence states are handed off by the chunk tiles' own hop
            a.relay = 0;
            a.slots = 1;
        }
        // initial state into the ring's slot 0; every sync word reset (chain counters to 1: the
        // state entering chunk 0 is ready -- in the relay form its relay waves publish it)
        // the 16-bit tile keeps p in its interleaved order; the fp32 tile in plain order.
        // Skipped without an initial state when the previous call on this workspace, the same
        // one, left the words reset (SSD_FLAG_WORKSPACE_READY).
        const int es = (int)elem_size(p->state_dtype), K = a.slots, pperm = p->in_dtype != SSD_F32;
        const int pw = ssd::p_per_wave(p->headdim);
        const uint32_t flag_init = a.relay ? 0u : 1u;
        const ReadyKey key = ready_key(p, workspace, a.relay, a.slots, l.nsync);
        const bool was_ready = ready_take(key);  // (the entry stays dropped until this call's copy-out)
        if (!(was_ready && (p->flags & SSD_FLAG_WORKSPACE_READY) && !initial_state && !seqst))
            e = ssd::launch_ring_copy(initial_state, a.states, 1, p->batch, p->nheads, p->headdim, pw, p->dstate, K,
                                      0, es, pperm, a.flags, l.nsync, l.nflags, (uint32_t)ssd::kChainStride,
                                      flag_init, ~(size_t)0, st);
        if (e == hipSuccess) e = mark(ev_begin);
        if (e == hipSuccess) e = dispatch(ssd::STEP_FUSED, p, a, st);
        if (e == hipSuccess) e = mark(ev_end);
        // final state out of the last chunk's slot (the relay form keeps it in slot 1), and every
        // sync word but the status word reset for the next call; with per-sequence states the
        // kernel wrote every final state itself
        if (e == hipSuccess && !seqst) {
            e = ssd::launch_ring_copy(a.states, final_state, 0, p->batch, p->nheads, p->headdim, pw, p->dstate, K,
                                      a.relay ? 1 : l.w.nchunks % K, es, pperm, a.flags, l.nsync, l.nflags,
                                      (uint32_t)ssd::kChainStride, flag_init, l.status_w, st);
            if (e == hipSuccess) ready_put(key);
        }
        return hip_status(e);
    }
    e = mark(ev_begin);
    if (e == hipSuccess) e = dispatch(ssd::STEP_CUMSUM, p, a, st);
    if (e == hipSuccess) e = dispatch(ssd::STEP_BMM, p, a, st);
    if (e == hipSuccess) e = dispatch(ssd::STEP_CHUNK_STATE, p, a, st);
    if (e == hipSuccess) e = boundary_in(p, l, a, initial_state, a.status, 1, 0, st);
    if (e == hipSuccess) e = ssd::launch_state_passing(a, p->headdim * p->dstate, st);
    if (e == hipSuccess && !seqst) e = boundary_out(p, l, a, final_state, st);
    if (e == hipSuccess) e = dispatch(ssd::STEP_CHUNK_SCAN, p, a, st);
    if (e == hipSuccess) e = mark(ev_end);
    return hip_status(e);
}

SSD_EXPORT ssd_status_t ssd_prefill(const ssd_params_t* p, const void* x, const void* dt, const float* A,
                                   const void* B, const void* C, const float* D, const float* dt_bias,
                                   const void* initial_state, void* y, void* final_state, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return ssd::prefill_impl(p, x, dt, A, B, C, D, dt_bias, initial_state, y, final_state, workspace, workspace_bytes,
                             stream, nullptr, nullptr, nullptr);
}

SSD_EXPORT ssd_status_t ssd_prefill_varlen(const ssd_params_t* p, const void* x, const void* dt, const float* A,
                                          const void* B, const void* C, const float* D, const float* dt_bias,
                                          const int32_t* seq_idx, const void* initial_state, void* y,
                                          void* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    if (!seq_idx) return SSD_ERR_NULL_POINTER;
    return ssd::prefill_impl(p, x, dt, A, B, C, D, dt_bias, initial_state, y, final_state, workspace, workspace_bytes,
                             stream, nullptr, nullptr, seq_idx);
}

SSD_EXPORT ssd_status_t ssd_prefill_varlen_states(const ssd_params_t* p, const void* x, const void* dt,
                                                 const float* A, const void* B, const void* C, const float* D,
                                                 const float* dt_bias, const int32_t* seq_idx, int nseq,
                                                 const void* initial_states, void* y, void* final_states,
                                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (!seq_idx || !final_states) return SSD_ERR_NULL_POINTER;
    if (nseq < 1) return SSD_ERR_INVALID_SHAPE;
    return ssd::prefill_impl(p, x, dt, A, B, C, D, dt_bias, nullptr, y, nullptr, workspace, workspace_bytes, stream,
                             nullptr, nullptr, seq_idx, ssd::SeqStates{initial_states, final_states, nseq});
}

SSD_EXPORT ssd_status_t ssd_prefill_timed(const ssd_params_t* p, const void* x, const void* dt, const float* A,
                                         const void* B, const void* C, const float* D, const float* dt_bias,
                                         const void* initial_state, void* y, void* final_state, void* workspace,
                                         size_t workspace_bytes, void* stream, void* kernel_begin,
                                         void* kernel_end) {
    if (!kernel_begin || !kernel_end) return SSD_ERR_NULL_POINTER;
    return ssd::prefill_impl(p, x, dt, A, B, C, D, dt_bias, initial_state, y, final_state, workspace, workspace_bytes,
                             stream, (hipEvent_t)kernel_begin, (hipEvent_t)kernel_end, nullptr);
}

SSD_EXPORT ssd_status_t ssd_check_device_status(const ssd_params_t* p, const void* workspace, void* stream) {
    ssd_status_t s = validate(p);
    if (s != SSD_OK) return s;
    if (!workspace) return SSD_ERR_NULL_POINTER;
    const Layout l = layout(p);
    uint32_t word = 0;
    hipStream_t st = (hipStream_t)stream;
    if (hipStreamSynchronize(st) != hipSuccess) return SSD_ERR_HIP;
    if (hipMemcpy(&word, (const char*)workspace + l.w.status_offset, 4, hipMemcpyDeviceToHost) != hipSuccess)
        return SSD_ERR_HIP;
    return word == 0 ? SSD_OK : (ssd_status_t)word;
}

// ---- the single-token decode step -----------------------------------------------------------

namespace {

ssd_status_t validate_decode(const ssd_params_t* p) {
    if (!p) return SSD_ERR_NULL_POINTER;
    if (p->struct_size < kParamsV1Size) return SSD_ERR_INVALID_ARGUMENT;
    if (p->in_dtype < SSD_F32 || p->in_dtype > SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
    if (p->state_dtype < SSD_F32 || p->state_dtype > SSD_BF16) return SSD_ERR_INVALID_ARGUMENT;
    if (p->dt_softplus != 0 && p->dt_softplus != 1) return SSD_ERR_INVALID_ARGUMENT;
    if (p->batch < 1 || p->seqlen != 1 || p->nheads < 1 || p->headdim < 1 || p->dstate < 1 || p->ngroups < 1)
        return SSD_ERR_INVALID_SHAPE;
    if (p->nheads % p->ngroups) return SSD_ERR_INVALID_SHAPE;
    const int N = p->dstate;
    if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return SSD_ERR_UNSUPPORTED;
    const int64_t rb = ssd::decode_rows_per_block(N);
    const int64_t blocks = (int64_t)p->batch * p->nheads * ((p->headdim + rb - 1) / rb);
    if (blocks >= (int64_t)1 << 31) return SSD_ERR_INVALID_SHAPE;
    return SSD_OK;
}

}  // namespace

SSD_EXPORT ssd_status_t ssd_decode_step(const ssd_params_t* p, const void* x, const void* dt, const float* A,
                                        const void* B, const void* C, const float* D, const float* dt_bias,
                                        const void* state_in, void* state_out, void* y, void* stream) {
    const ssd_status_t s = validate_decode(p);
    if (s != SSD_OK) return s;
    if (!x || !dt || !A || !B || !C || !state_out || !y) return SSD_ERR_NULL_POINTER;
    const size_t es = elem_size(p->in_dtype);
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) || !aligned(state_out, 16) ||
        !aligned(state_in, 16) || !aligned(dt, es) || !aligned(A, 4) || !aligned(D, 4) || !aligned(dt_bias, 4))
        return SSD_ERR_MISALIGNED;
    ssd::DecodeArgs a{};
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.D = D;
    a.dt_bias = dt_bias;
    a.state_in = state_in;
    a.state_out = state_out;
    a.y = y;
    a.batch = p->batch;
    a.nheads = p->nheads;
    a.headdim = p->headdim;
    a.dstate = p->dstate;
    a.ngroups = p->ngroups;
    a.state_dtype = p->state_dtype;
    a.softplus = p->dt_softplus;
    return hip_status(ssd::launch_decode(a, p->in_dtype, (hipStream_t)stream));
}

// ---- the Mamba-2 block around the SSD: convolution before, gated norm after ----------------

namespace {

bool is16(const ssd_params_t* p) { return p->in_dtype == SSD_F16 || p->in_dtype == SSD_BF16; }

// Workspace of ssd_prefill_block: the SSD's own layout, then (fused) the norm's per-token sums
// and per-(b, c, g) tile counts appended to the sync words (so the copy-in launch clears them),
// then the convolved B and C (and x for the unfused form) and y.
struct BlockLayout {
    Layout l;
    size_t nsum_w, ncount_w, nsync_total;
    size_t x_off, b_off, c_off, y_off, total;
};

BlockLayout block_layout(const ssd_params_t* p) {
    BlockLayout k{};
    k.l = layout(p);
    const size_t B = p->batch, L = p->seqlen, H = p->nheads, P = p->headdim, N = p->dstate, G = p->ngroups;
    const size_t es = elem_size(p->in_dtype), nc = k.l.w.nchunks;
    const bool fused = p->impl == SSD_IMPL_FUSED;
    k.nsum_w = k.l.nsync;
    k.ncount_w = k.nsum_w + (fused ? B * L * G : 0);
    k.nsync_total = k.ncount_w + (fused ? B * nc * G : 0);
    size_t off = align_up(k.l.w.sync_offset + 4 * k.nsync_total);
    if (off < k.l.w.total_bytes) off = k.l.w.total_bytes;
    k.x_off = off;
    off = align_up(off + (fused ? 0 : B * L * H * P * es));
    k.b_off = off;
    off = align_up(off + B * L * G * N * es);
    k.c_off = off;
    off = align_up(off + B * L * G * N * es);
    k.y_off = off;
    off = align_up(off + B * L * H * P * es);
    k.total = off;
    return k;
}

ssd_status_t validate_block(const ssd_params_t* p) {
    ssd_status_t s = validate(p);
    if (s != SSD_OK) return s;
    if (!is16(p)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// The fused block form takes P, N in {64, 128} and tiles that never straddle two groups.
bool block_fusable(const ssd_params_t* p) {
    const int P = p->headdim, N = p->dstate;
    if ((P != 64 && P != 128) || (N != 64 && N != 128)) return false;
    return (p->nheads / p->ngroups) % ssd::heads_per_tile(P) == 0;
}

hipError_t launch_block(int step, const ssd_params_t* p, ssd::SsdArgs& a, hipStream_t st) {
    if (p->in_dtype == SSD_F16) return ssd::launch_block_f16(step, p->headdim, p->dstate, p->chunk_size, a, st);
    return ssd::launch_block_bf16(step, p->headdim, p->dstate, p->chunk_size, a, st);
}

}  // namespace

SSD_EXPORT size_t ssd_prefill_block_workspace_size(const ssd_params_t* p) {
    if (validate_block(p) != SSD_OK) return 0;
    return block_layout(p).total;
}

SSD_EXPORT ssd_status_t ssd_conv_silu(const ssd_params_t* p, const void* xbc, const float* conv_w,
                                      const float* conv_b, const void* conv_state, void* x, void* B, void* C,
                                      void* stream) {
    ssd_status_t s = validate_block(p);
    if (s != SSD_OK) return s;
    if (!xbc || !conv_w || !x || !B || !C) return SSD_ERR_NULL_POINTER;
    if (!aligned(xbc, 16) || !aligned(conv_w, 16) || !aligned(conv_b, 4) || !aligned(conv_state, 2) ||
        !aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16))
        return SSD_ERR_MISALIGNED;
    ssd::ConvArgs a{xbc, conv_w, conv_b, conv_state, x, B, C, p->batch, p->seqlen, p->nheads * p->headdim,
                    p->ngroups * p->dstate};
    return hip_status(ssd::launch_conv_silu(a, p->in_dtype, (hipStream_t)stream));
}

SSD_EXPORT ssd_status_t ssd_gated_norm(const ssd_params_t* p, const void* y, const void* z, const float* norm_w,
                                       float norm_eps, void* out, void* stream) {
    ssd_status_t s = validate_block(p);
    if (s != SSD_OK) return s;
    if (!y || !z || !norm_w || !out) return SSD_ERR_NULL_POINTER;
    if (!aligned(y, 16) || !aligned(z, 16) || !aligned(norm_w, 16) || !aligned(out, 16)) return SSD_ERR_MISALIGNED;
    if (!(norm_eps >= 0.f)) return SSD_ERR_INVALID_ARGUMENT;
    ssd::NormArgs a{y, z, norm_w, out, (int64_t)p->batch * p->seqlen, p->nheads * p->headdim, p->ngroups, norm_eps};
    return hip_status(ssd::launch_gated_norm(a, p->in_dtype, (hipStream_t)stream));
}

SSD_EXPORT ssd_status_t ssd_prefill_block(const ssd_params_t* p, const void* xbc, const float* conv_w,
                                          const float* conv_b, const void* conv_state, const void* dt,
                                          const float* A, const float* D, const float* dt_bias, const void* z,
                                          const float* norm_w, float norm_eps, const void* initial_state, void* out,
                                          void* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    ssd_status_t s = validate_block(p);
    if (s != SSD_OK) return s;
    const bool fused = p->impl == SSD_IMPL_FUSED;
    if (fused && !block_fusable(p)) return SSD_ERR_UNSUPPORTED;
    if (!xbc || !conv_w || !dt || !A || !z || !norm_w || !out || !final_state || !workspace) return SSD_ERR_NULL_POINTER;
    if (!aligned(xbc, 16) || !aligned(conv_w, 16) || !aligned(conv_b, 4) || !aligned(conv_state, 2) ||
        !aligned(dt, 2) || !aligned(A, 4) || !aligned(D, 4) || !aligned(dt_bias, 4) || !aligned(z, 16) ||
        !aligned(norm_w, 16) || !aligned(initial_state, 16) || !aligned(out, 16) || !aligned(final_state, 16) ||
        !aligned(workspace, kAlign))
        return SSD_ERR_MISALIGNED;
    if (!(norm_eps >= 0.f)) return SSD_ERR_INVALID_ARGUMENT;
    const BlockLayout k = block_layout(p);
    if (workspace_bytes < k.total) return SSD_ERR_WORKSPACE_TOO_SMALL;
    ready_drop(workspace);  // this form always resets the sync words itself
    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    const size_t HP = (size_t)p->nheads * p->headdim, GN = (size_t)p->ngroups * p->dstate;
    void* yw = ws + k.y_off;
    if (!fused) {
        // the three steps as separate launches: conv -> the five SSD kernels -> norm
        ssd_status_t r = ssd_conv_silu(p, xbc, conv_w, conv_b, conv_state, ws + k.x_off, ws + k.b_off, ws + k.c_off,
                                       stream);
        if (r == SSD_OK)
            r = ssd::prefill_impl(p, ws + k.x_off, dt, A, ws + k.b_off, ws + k.c_off, D, dt_bias, initial_state, yw,
                                  final_state, workspace, k.l.w.total_bytes, stream, nullptr, nullptr, nullptr);
        if (r == SSD_OK) r = ssd_gated_norm(p, yw, z, norm_w, norm_eps, out, stream);
        return r;
    }
    const Layout& l = k.l;
    ssd::SsdArgs a = make_args(p, l, workspace);
    a.x = xbc;
    a.x_stride = (int)(HP + 2 * GN);
    a.xbc = xbc;
    a.xbc_hp = (int)HP;
    a.conv_w = conv_w;
    a.conv_b = conv_b;
    a.conv_state = conv_state;
    a.dt = dt;
    a.A = A;
    a.B = ws + k.b_off;
    a.C = ws + k.c_off;
    a.D = D;
    a.dt_bias = dt_bias;
    a.y = yw;
    a.z = z;
    a.norm_w = norm_w;
    a.norm_eps = norm_eps;
    a.nsum = (float*)(ws + l.w.sync_offset) + k.nsum_w;
    a.ncount = (uint32_t*)(ws + l.w.sync_offset) + k.ncount_w;
    a.out = out;
    a.has_h0 = initial_state != nullptr;
    DevInfo d;
    hipError_t e = device_info(&d);
    if (e == hipSuccess) e = launch_block(ssd::STEP_FUSED_OCCUPANCY, p, a, st);
    if (e != hipSuccess) return hip_status(e);
    set_partitions(p, l, d, a);
    // The norm kernel after the launch is the default (measured faster on MI355X than every
    // in-launch form tried).  MAMBA_SSD_BLOCK_NORM=1 runs the norm inside the launch instead,
    // where every (b, g) pair's tiles share one partition (one XCD's L2 holds the rows and sums
    // the norm items read back): the chunk tiles then pass the state themselves and claim whole
    // pairs together, and a norm item waits only on chunk tiles with smaller tickets.
    bool aligned_parts = true;
    for (int x = 0; x <= a.nparts; ++x) aligned_parts = aligned_parts && a.part_u0[x] % l.tpg == 0;
    a.norm_fused = (aligned_parts && env_int("MAMBA_SSD_BLOCK_NORM", 0) == 1) ? 1 : 0;
    if (a.norm_fused) {
        a.relay = 0;
        a.slots = 1;
        a.chain_group = 0;
    }
    const int es = (int)elem_size(p->state_dtype), K = a.slots, pperm = 1;
    const int pw = ssd::p_per_wave(p->headdim);
    e = ssd::launch_ring_copy(initial_state, a.states, 1, p->batch, p->nheads, p->headdim, pw, p->dstate, K, 0, es,
                              pperm, a.flags, k.nsync_total, l.nflags, (uint32_t)ssd::kChainStride,
                              a.relay ? 0u : 1u, ~(size_t)0, st);
    if (e == hipSuccess) e = launch_block(ssd::STEP_FUSED, p, a, st);
    if (e == hipSuccess)
        e = ssd::launch_ring_copy(a.states, final_state, 0, p->batch, p->nheads, p->headdim, pw, p->dstate, K,
                                  a.relay ? 1 : l.w.nchunks % K, es, pperm, nullptr, 0, 0, 1, 0u, ~(size_t)0, st);
    if (e != hipSuccess) return hip_status(e);
    if (!a.norm_fused) return ssd_gated_norm(p, yw, z, norm_w, norm_eps, out, stream);
    return SSD_OK;
}
