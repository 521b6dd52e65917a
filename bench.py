"""Benchmark: Mamba-2 SSD chunked prefill on one MI355X.

    python bench.py [--steps K] [--warmup W] [--chunk Q] [--workload NAME] [--no-cpu-baseline]

A step is one ssd_prefill call (the whole hot path: boundary copies + the fused SSD
kernel) over one batch of seeded synthetic inputs already resident in HBM.  Prints ONE
JSON line with tokens/s, the roofline of the fused kernel (timed live with HIP events
the library records around it), the unfused five-kernel form timed the same way, a
chunk-size sweep, and the fp64 CPU oracle timed on a bounded sample.

Roofline bytes are the algorithmic HBM traffic of the chunked method: the compulsory
traffic (read x, dt, B, C, the initial state and the per-head parameters once; write y and
the final state once) plus one write and one read of every inter-chunk state, the same
for both forms.  The compulsory-only figure is reported alongside ("achieved_compulsory").
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
METRIC = "SSD prefill tokens/s per layer + % HBM/MFMA roofline (fused vs unfused)"
ESZ = {"f32": 4, "f16": 2, "bf16": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, Q, has_h0):
    """Compulsory bytes, state-exchange bytes and causal flops of one call."""
    B, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    e, es = ESZ[w.dtype], ESZ[w.state_dtype]
    T = B * L
    nc = -(-L // Q)
    compulsory = T * (2 * H * P * e + H * e + 2 * G * N * e) + (2 if has_h0 else 1) * B * H * P * N * es + 3 * H * 4
    exchange = 2 * B * nc * H * P * N * es
    flops = T * (G * (Q + 1) * N + H * ((Q + 1) * P + 4 * P * N + 2 * P))
    return compulsory, exchange, flops


def measured_traffic(workload, Q):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "ssd_fused_%s_q%d_traffic.json" % (workload, Q))
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from mamba_ssd_prefill_amd.build import source_hash
    if t.get("kernel_source_hash") != source_hash():
        return None
    return t.get("bytes_per_launch")


def time_impl(ssd, torch, g, w, Q, impl, steps, warmup, state_dtype=None, relaxed=False):
    """Warm up, then time `steps` calls; returns (ms per call, mean kernel ms)."""
    sd_name = state_dtype or w.state_dtype
    prm = ssd.make_params(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, Q, w.dtype,
                          sd_name, True, impl, relaxed)
    ws = ssd.alloc_workspace(prm, g.x.device)
    y = torch.empty_like(g.x)
    sdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[sd_name]
    fin = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, dtype=sdt, device=g.x.device)
    h0 = g.h0.to(sdt) if g.h0 is not None else None
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

    used = []  # the workspace is reused untouched from call to call (SSD_FLAG_WORKSPACE_READY)

    def call(ev=None):
        ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, h0, chunk_size=Q, impl=impl,
                        state_dtype=sdt, workspace=ws, y=y, final_state=fin, kernel_events=ev, relaxed=relaxed,
                        workspace_ready=bool(used))
        used.append(1)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    kms = sum(a.elapsed_time(b) for a, b in evs) / steps
    status = ssd.check_device_status(prm, ws)
    if status != 0:
        raise RuntimeError("device status %d after %s Q=%d" % (status, impl, Q))
    del ws, y, fin
    return wall, kms


# warmup calls of each auxiliary leg (chunk sweep, fp16 state, precision points): each switches
# kernels and buffers, and its first few calls run slower than the steady state
SWEEP_WARMUP = 10


def settle(ssd, torch, g, w, Q, seconds):
    """Untimed fused and unfused calls, alternating, for about `seconds` before anything is
    timed: a fresh process's first ~25 calls run up to 8 % slower (measured on MI355X: clocks
    and first use of the buffers), so without this the first timed form would be measured
    during that ramp and the second after it.  Both forms are then timed at steady state, after
    their own warmup steps."""
    sdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.state_dtype]
    h0 = g.h0.to(sdt) if g.h0 is not None else None
    y = torch.empty_like(g.x)
    fin = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, dtype=sdt, device=g.x.device)
    wss = {}
    for impl in ("fused", "unfused"):
        prm = ssd.make_params(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, Q, w.dtype,
                              w.state_dtype, True, impl)
        wss[impl] = ssd.alloc_workspace(prm, g.x.device)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for impl in ("fused", "unfused"):
            ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, h0, chunk_size=Q, impl=impl,
                            state_dtype=sdt, workspace=wss[impl], y=y, final_state=fin)
        torch.cuda.synchronize()
    del wss, y, fin


def decode_bytes(w, batch):
    """Algorithmic HBM bytes of one decode step: the state read and written once, x, dt, B, C
    read and y written once, and the per-head parameters."""
    e, es = ESZ[w.dtype], ESZ[w.state_dtype]
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    return 2 * batch * H * P * N * es + batch * (2 * H * P * e + H * e + 2 * G * N * e) + 3 * H * 4


def time_decode(ssd, torch, w, batch, steps):
    """`steps` consecutive ssd_decode_step calls (one token per batch row each, a new token per
    step, the state updated in place) captured in one HIP graph and replayed, bracketed by HIP
    events on the replay stream; returns microseconds per step.  The graph keeps the host out of
    the timed region, as a decode loop on the device would."""
    gen = torch.Generator().manual_seed(77)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    dev = "cuda:0"
    x = torch.randn(steps, batch, H, P, generator=gen).to(tdt[w.dtype]).to(dev)
    dt = torch.randn(steps, batch, H, generator=gen).to(tdt[w.dtype]).to(dev)
    Bm = (torch.randn(steps, batch, G, N, generator=gen) / N ** 0.5).to(tdt[w.dtype]).to(dev)
    Cm = (torch.randn(steps, batch, G, N, generator=gen) / N ** 0.5).to(tdt[w.dtype]).to(dev)
    A = (-torch.exp(torch.rand(H, generator=gen) * 2.77)).to(dev)
    D = torch.randn(H, generator=gen).to(dev)
    bias = torch.full((H,), -4.0).to(dev)
    state = (0.1 * torch.randn(batch, H, P, N, generator=gen)).to(tdt[w.state_dtype]).to(dev)
    ys = torch.empty(steps, batch, H, P, dtype=tdt[w.dtype], device=dev)

    def run():
        for i in range(steps):
            ssd.ssd_decode_step(x[i], dt[i], A, Bm[i], Cm[i], D, bias, state, y=ys[i])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    graph.replay()
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * steps)


def decode_legs(ssd, torch, w, only_batch=0):
    """The decode step at the workload's layer shape, at its batch and at 16 times it (or at
    `only_batch` alone)."""
    dec = {}
    for bsz in ((only_batch,) if only_batch else (w.batch, 16 * w.batch)):
        log("decode step, batch %d" % bsz)
        us = time_decode(ssd, torch, w, bsz, 100 if bsz <= w.batch else 20)
        nb = decode_bytes(w, bsz)
        dec["batch%d" % bsz] = {"us_per_step": us, "tokens_per_s": bsz / (us / 1e6), "bytes": nb,
                                "achieved_gbs": nb / (us / 1e6) / 1e9, "frac": nb / (us / 1e6) / 1e9 / HBM_PEAK_GBS}
    return {"kernel": "k_decode", "bound": "hbm", "peak_gbs": HBM_PEAK_GBS, "copy_gbs": copy_bandwidth(torch),
            "state_dtype": w.state_dtype, "timing": "HIP events around replays of a HIP graph of consecutive steps",
            **dec}


def time_varlen(ssd, torch, steps):
    """The many-short-sequences workload (32 sequences of 1024 tokens, H=128, G=8, bf16, Q=128)
    two ways: as a batch of 32 rows, and packed into one row of 32768 tokens told apart by
    seq_idx (ssd_prefill_varlen).  Same tokens, same work; returns ms per call of each, fused."""
    from mamba_ssd_prefill_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["short_g8_bf16"]
    inp = workload_inputs(w)
    g = inp.to("cuda:0")
    Bt, L = w.batch, w.seqlen
    packed = [t.reshape(1, Bt * L, *t.shape[2:]) for t in (g.x, g.dt, g.B, g.C)]
    seq = torch.arange(Bt, dtype=torch.int32, device="cuda:0").repeat_interleave(L).reshape(1, Bt * L).contiguous()
    res = {}
    for name, args, kw in (("batched", (g.x, g.dt, g.A, g.B, g.C), {}),
                           ("packed", (packed[0], packed[1], g.A, packed[2], packed[3]), {"seq_idx": seq})):
        x = args[0]
        prm = ssd.make_params(x.shape[0], x.shape[1], w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size,
                              w.dtype, "f32", True, "fused")
        ws = ssd.alloc_workspace(prm, x.device)
        y = torch.empty_like(x)
        fin = torch.empty(x.shape[0], w.nheads, w.headdim, w.dstate, dtype=torch.float32, device=x.device)

        used = []

        def call():
            ssd.ssd_prefill(*args, g.D, g.dt_bias, None, chunk_size=w.chunk_size, impl="fused", workspace=ws,
                            y=y, final_state=fin, workspace_ready=bool(used), **kw)
            used.append(1)

        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        if ssd.check_device_status(prm, ws) != 0:
            raise RuntimeError("device status after the %s short-sequence run" % name)
        res[name] = e0.elapsed_time(e1) / steps
    tokens = Bt * L
    return {"workload": "32 sequences x 1024 tokens, H=128, P=64, N=128, G=8, bf16, Q=128",
            "batched_ms": res["batched"], "packed_ms": res["packed"],
            "batched_tokens_per_s": tokens / (res["batched"] / 1e3),
            "packed_tokens_per_s": tokens / (res["packed"] / 1e3)}


def time_block(ssd, torch, steps):
    """The block form at the 2.7B layer shape (B=8, L=8192, H=80, P=64, N=128, G=1, Q=128, bf16,
    fp32 state, initial state): the width-4 convolution before and the gated norm after the SSD.
    Three ways, ms per call each: fused (one launch plus the boundary copies; the norm inside the
    launch), separate (the conv kernel, the fused SSD, the norm kernel) and unfused (the conv
    kernel, the five SSD kernels, the norm kernel).  Bytes: the fused block reads xBC, dt and z
    and writes out once (plus the states); the separate form also writes and re-reads the
    convolved x, B, C and y."""
    from mamba_ssd_prefill_amd.inputs import WORKLOADS, make_block_inputs, workload_inputs
    w = WORKLOADS["mamba2_2p7b_bf16"]
    B_, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, 128
    g = workload_inputs(w).to("cuda:0")
    b = make_block_inputs(B_, L, H, P, N, G, dtype=w.dtype, has_state=False, seed=2003).to("cuda:0")
    eps = 1e-5
    T, e, hp, gn = B_ * L, ESZ[w.dtype], H * P, G * N
    comp, exch, _ = algorithmic(w, Q, True)
    fused_bytes = comp + exch + T * (2 * gn * e + hp * e)  # xBC instead of x, B, C: + z read; out replaces y
    separate_bytes = fused_bytes + 2 * T * (hp + 2 * gn) * e + 2 * T * hp * e
    out = torch.empty(B_, L, hp, dtype=b.xbc.dtype, device="cuda:0")
    fin = torch.empty(B_, H, P, N, dtype=torch.float32, device="cuda:0")
    res = {}
    prm_f = ssd.make_params(B_, L, H, P, N, G, Q, w.dtype, "f32", True, "fused")
    prm_u = ssd.make_params(B_, L, H, P, N, G, Q, w.dtype, "f32", True, "unfused")
    ws_f = torch.empty(ssd.block_workspace_size(prm_f), dtype=torch.uint8, device="cuda:0")
    ws_u = torch.empty(ssd.block_workspace_size(prm_u), dtype=torch.uint8, device="cuda:0")
    ws_s = ssd.alloc_workspace(prm_f, "cuda:0")
    x = torch.empty(B_, L, H, P, dtype=b.xbc.dtype, device="cuda:0")
    Bm = torch.empty(B_, L, G, N, dtype=b.xbc.dtype, device="cuda:0")
    Cm = torch.empty_like(Bm)
    y = torch.empty_like(x)
    kw = dict(nheads=H, headdim=P, ngroups=G, dstate=N, chunk_size=Q)

    def fused():
        ssd.ssd_prefill_block(b.xbc, b.conv_w, b.conv_b, None, g.dt, g.A, g.D, g.dt_bias, b.z, b.norm_w, eps, g.h0,
                              impl="fused", workspace=ws_f, out=out, final_state=fin, **kw)

    def unfused():
        ssd.ssd_prefill_block(b.xbc, b.conv_w, b.conv_b, None, g.dt, g.A, g.D, g.dt_bias, b.z, b.norm_w, eps, g.h0,
                              impl="unfused", workspace=ws_u, out=out, final_state=fin, **kw)

    lib = ssd.load_library()
    import ctypes

    def separate():
        st = ssd._stream(torch.device("cuda:0"))
        ssd._check(lib.ssd_conv_silu(ctypes.byref(prm_f), ssd._ptr(b.xbc), ssd._ptr(b.conv_w), ssd._ptr(b.conv_b),
                                     None, ssd._ptr(x), ssd._ptr(Bm), ssd._ptr(Cm), st), "ssd_conv_silu")
        ssd.ssd_prefill(x, g.dt, g.A, Bm, Cm, g.D, g.dt_bias, g.h0, chunk_size=Q, impl="fused", workspace=ws_s, y=y,
                        final_state=fin)
        ssd._check(lib.ssd_gated_norm(ctypes.byref(prm_f), ssd._ptr(y), ssd._ptr(b.z), ssd._ptr(b.norm_w),
                                      ctypes.c_float(eps), ssd._ptr(out), st), "ssd_gated_norm")

    for name, fn in (("fused", fused), ("separate", separate), ("unfused", unfused)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    if ssd.check_device_status(prm_f, ws_f) != 0:
        raise RuntimeError("device status after the fused block run")
    r = {"workload": "2.7B layer shape, conv (width 4) + SSD + gated norm, bf16, Q=128",
         "fused_ms": res["fused"], "separate_ms": res["separate"], "unfused_ms": res["unfused"],
         "fused_tokens_per_s": T / (res["fused"] / 1e3), "separate_tokens_per_s": T / (res["separate"] / 1e3),
         "speedup_fused_vs_separate": res["separate"] / res["fused"],
         "bytes_fused": fused_bytes, "bytes_separate": separate_bytes,
         "frac_fused": fused_bytes / (res["fused"] / 1e3) / 1e9 / HBM_PEAK_GBS,
         "frac_separate": separate_bytes / (res["separate"] / 1e3) / 1e9 / HBM_PEAK_GBS}
    return r


def copy_bandwidth(torch):
    """Bytes read plus written per second of a 512 MiB device-to-device copy (torch's copy
    kernel): what a plain streaming kernel reaches on this device, for context."""
    src = torch.empty(1 << 27, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2 * src.numel() * 4 / (e0.elapsed_time(e1) / 10 / 1e3) / 1e9


def cpu_baseline(inp, w, seconds):
    """The fp64 oracle (as it stands) on whole (batch, head) chains of the same inputs,
    `threads` chains per call, until ~`seconds` have passed (whole passes repeat)."""
    import oracle
    threads = oracle.num_threads()
    pairs = [(b, h) for b in range(w.batch) for h in range(w.nheads)]
    done, t0 = 0, time.perf_counter()
    while True:
        k = done % len(pairs)
        oracle.recurrence(**inp.args(), bh=pairs[k:k + threads])
        done += len(pairs[k:k + threads])
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    layer_tokens = done * w.seqlen / w.nheads  # one layer token = all H heads of one (b, t)
    return {"value": layer_tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d (batch, head) chains of the %d in the workload (%.2f passes), %d tokens each, "
                      "fp64 recurrence with y stored, %.1f s" % (done, len(pairs), done / len(pairs), w.seqlen, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle", type=float, default=0.25,
                    help="seconds of untimed fused and unfused calls before the first timed form (0: none)")
    ap.add_argument("--workload", default="mamba2_2p7b_bf16")
    ap.add_argument("--chunk", type=int, default=0, help="chunk size (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode-step legs (for a kernel trace of k_decode); prints their JSON")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="with --decode-only: this batch size only (default: the workload's and 16 times it)")
    ap.add_argument("--block-only", action="store_true",
                    help="only the block-form leg (convolution + SSD + gated norm; for a kernel trace); prints its JSON")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 --pmc: a 1 GiB device copy (counter calibration), "
                         "then --steps fused calls; prints nothing")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SSD prefill here is a single-GPU kernel and no "
              "multi-GPU path is built (see DESIGN.md for how it would shard); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mamba_ssd_prefill_amd as ssd
    from mamba_ssd_prefill_amd.inputs import WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    ssd.load_library()
    w = WORKLOADS[args.workload]
    Q = args.chunk or w.chunk_size
    if args.decode_only:
        print(json.dumps(decode_legs(ssd, torch, w, args.decode_batch)), flush=True)
        return
    if args.block_only:
        print(json.dumps(time_block(ssd, torch, args.steps)), flush=True)
        return
    log("generating %s inputs" % w.name)
    inp = workload_inputs(w)
    g = inp.to("cuda:0")
    torch.cuda.synchronize()

    if args.counters:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)  # 1 GiB read + 1 GiB written per copy
        torch.cuda.synchronize()
        del src, dst
        sdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.state_dtype]
        for impl in ("fused", "unfused"):
            for _ in range(args.steps):
                ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q, impl=impl,
                                state_dtype=sdt)
            torch.cuda.synchronize()
        return

    log("settling (%.2f s of untimed fused and unfused calls)" % args.settle)
    settle(ssd, torch, g, w, Q, args.settle)
    log("timing fused Q=%d" % Q)
    f_wall, f_kms = time_impl(ssd, torch, g, w, Q, "fused", args.steps, args.warmup)
    log("timing unfused Q=%d" % Q)
    u_wall, u_kms = time_impl(ssd, torch, g, w, Q, "unfused", args.steps, args.warmup)

    comp, exch, flops = algorithmic(w, Q, inp.h0 is not None)
    tokens = w.batch * w.seqlen
    k_s = f_kms / 1e3
    traffic = measured_traffic(w.name, Q)
    alg = comp + exch
    roof = {"bound": "hbm", "achieved": alg / k_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": alg / k_s / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
            # the HBM bytes the counters measured (when taken on these sources) over the same time
            "frac_measured": (traffic / k_s / 1e9 / HBM_PEAK_GBS) if traffic else None,
            "kernel": "k_fused16" if w.dtype != "f32" else "k_fused", "kernel_ms": f_kms,
            "bytes_per_launch": alg, "compulsory_bytes": comp, "state_exchange_bytes": exch,
            "achieved_compulsory": comp / k_s / 1e9, "frac_compulsory": comp / k_s / 1e9 / HBM_PEAK_GBS,
            "mfma_tflops": flops / k_s / 1e12,
            "mfma_frac": flops / k_s / 1e12 / MFMA_PEAK_TFLOPS[w.dtype]}
    out = {
        "metric": METRIC, "value": tokens / (f_wall / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": f_wall, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups, "chunk_size": Q,
                   "state_dtype": w.state_dtype, "initial_state": inp.h0 is not None, "impl": "fused",
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "unfused": {"ms_per_step": u_wall, "value": tokens / (u_wall / 1e3), "kernels_ms": u_kms,
                    "frac": alg / (u_kms / 1e3) / 1e9 / HBM_PEAK_GBS,
                    "frac_compulsory": comp / (u_kms / 1e3) / 1e9 / HBM_PEAK_GBS,
                    "mfma_tflops": flops / (u_kms / 1e3) / 1e12,
                    "mfma_frac": flops / (u_kms / 1e3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype]},
        "speedup_fused_vs_unfused": u_wall / f_wall,
        "settle_s": args.settle,
    }
    if not args.no_sweep:
        sweep = {}
        for q in (w.chunk_sweep or (Q,)):
            if q == Q:
                sweep[str(q)] = {"fused_ms": f_wall, "unfused_ms": u_wall}
                continue
            log("sweep Q=%d" % q)
            fw, fk = time_impl(ssd, torch, g, w, q, "fused", max(10, args.steps // 2), SWEEP_WARMUP)
            uw, uk = time_impl(ssd, torch, g, w, q, "unfused", max(10, args.steps // 2), SWEEP_WARMUP)
            sweep[str(q)] = {"fused_ms": fw, "unfused_ms": uw, "fused_kernel_ms": fk}
        for q, v in sweep.items():
            # the roofline fraction of the fused kernel at this chunk size (its own algorithmic bytes)
            c_q, x_q, _ = algorithmic(w, int(q), inp.h0 is not None)
            v["frac"] = (c_q + x_q) / (v.get("fused_kernel_ms", f_kms) / 1e3) / 1e9 / HBM_PEAK_GBS
        out["chunk_sweep"] = sweep
        if w.state_dtype == "f32" and w.dtype != "f32":
            # the same call with the inter-chunk states (and h0 / final state) stored in fp16
            log("fp16 state Q=%d" % Q)
            hw, hk = time_impl(ssd, torch, g, w, Q, "fused", max(10, args.steps // 2), SWEEP_WARMUP, state_dtype="f16")
            c16, x16, _ = algorithmic(w.with_(state_dtype="f16"), Q, inp.h0 is not None)
            out["state_f16"] = {"fused_ms": hw, "fused_kernel_ms": hk, "value": tokens / (hw / 1e3),
                                "frac": (c16 + x16) / (hk / 1e3) / 1e9 / HBM_PEAK_GBS}
            # exact vs relaxed intermediates x fp32 vs fp16 state storage, at Q = 128 and 256
            # (the pages' precision / performance trade-off), fused form
            prec = {}
            for q in (128, 256):
                for sd in ("f32", "f16"):
                    for rel in (False, True):
                        key = "q%d_%s_%s" % (q, sd, "relaxed" if rel else "exact")
                        if q == Q and sd == w.state_dtype and not rel:
                            prec[key] = {"fused_ms": f_wall, "fused_kernel_ms": f_kms}
                            continue
                        log("precision point %s" % key)
                        pw, pk = time_impl(ssd, torch, g, w, q, "fused", max(10, args.steps // 2), SWEEP_WARMUP,
                                           state_dtype=sd, relaxed=rel)
                        prec[key] = {"fused_ms": pw, "fused_kernel_ms": pk}
            for key, v in prec.items():
                v["value"] = tokens / (v["fused_ms"] / 1e3)
            out["precision_sweep"] = prec
        log("packed variable-length input")
        out["varlen"] = time_varlen(ssd, torch, 10)
        log("conv + SSD + norm block")
        out["block"] = time_block(ssd, torch, 10)
        out["decode"] = decode_legs(ssd, torch, w)
    del g
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
