"""Helpers shared by the GPU parity tests: run the HIP path, compare with the oracle."""
import contextlib
import os
import sys

import numpy as np
import torch

import mamba_ssd_prefill_amd as ssd
import oracle
from parity import StreamGate, gate

DT_NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU; none is visible")
    ssd.load_library()  # raises if the HIP library is not built: no fallback exists
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_STATE_CODE = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


@contextlib.contextmanager
def fused_form(impl):
    """impl "fused_hop" / "fused_relay" / "fused_relay2" / "fused_relay4": the fused form with
    the chunk tiles' own state hop / with relay items (MAMBA_SSD_RELAY = 0 / 1, or 2 / 4 relay
    waves per chain part); "fused" and "unfused" leave the choice to the library.  Yields the
    impl name the binding takes."""
    old = os.environ.pop("MAMBA_SSD_RELAY", None)
    forms = {"fused_hop": "0", "fused_relay": "1", "fused_relay2": "2", "fused_relay4": "4"}
    if impl in forms:
        os.environ["MAMBA_SSD_RELAY"] = forms[impl]
    try:
        yield "fused" if impl.startswith("fused") else impl
    finally:
        os.environ.pop("MAMBA_SSD_RELAY", None)
        if old is not None:
            os.environ["MAMBA_SSD_RELAY"] = old


def run_gpu(inp, chunk_size, impl, state_dtype=None, dev="cuda:0", relaxed=False):
    """One ssd_prefill on the GPU; also requires the device status word to read SSD_OK."""
    with fused_form(impl) as name:
        return _run_gpu(inp, chunk_size, name, state_dtype, dev, relaxed)


def _run_gpu(inp, chunk_size, impl, state_dtype, dev, relaxed=False):
    g = inp.to(dev)
    if state_dtype is None:
        state_dtype = g.h0.dtype if g.h0 is not None else torch.float32
    Bt, L, H, P = g.x.shape
    G, N = g.B.shape[2], g.B.shape[3]
    prm = ssd.make_params(Bt, L, H, P, N, G, chunk_size, DT_NAME[g.x.dtype], _STATE_CODE[state_dtype],
                          inp.dt_softplus, impl, relaxed)
    ws = ssd.alloc_workspace(prm, g.x.device)
    y, fin = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=chunk_size,
                             impl=impl, dt_softplus=inp.dt_softplus,
                             state_dtype=state_dtype, workspace=ws, relaxed=relaxed)
    torch.cuda.synchronize()
    status = ssd.check_device_status(prm, ws)
    assert status == 0, "device status %d after %s Q=%d" % (status, impl, chunk_size)
    return y, fin


def f64(t):
    return None if t is None else t.detach().cpu().to(torch.float64).numpy()


def check_full(inp, y, fin, name=""):
    """Every element of y and the final state against the fp64 recurrence."""
    yr, fr = oracle.recurrence_full(**inp.args())
    in_dt = DT_NAME[inp.x.dtype]
    st_dt = DT_NAME[fin.dtype]
    skip = (f64(inp.D)[None, None, :, None] * f64(inp.x)) if inp.D is not None else None
    r1 = gate(f64(y), yr, in_dt, in_dt, skip=skip, name=name + " y")
    r2 = gate(f64(fin), fr, st_dt, in_dt, name=name + " final")
    return r1, r2


def check_sampled(inp, y, fin, pairs, name=""):
    """The chains (b, h) in `pairs`, all tokens, against the fp64 recurrence."""
    yr, fr, _ = oracle.recurrence(**inp.args(), bh=pairs)
    in_dt = DT_NAME[inp.x.dtype]
    st_dt = DT_NAME[fin.dtype]
    ys = np.stack([f64(y[b, :, h]) for (b, h) in pairs])
    fs = np.stack([f64(fin[b, h]) for (b, h) in pairs])
    skip = None
    if inp.D is not None:
        skip = np.stack([float(inp.D[h]) * f64(inp.x[b, :, h]) for (b, h) in pairs])
    r1 = gate(ys, yr, in_dt, in_dt, skip=skip, name=name + " y")
    r2 = gate(fs, fr, st_dt, in_dt, name=name + " final")
    return r1, r2


def check_all_chains(inp, y, fin, name="", heads_per_block=0):
    """Every element of y and of the final state against the fp64 recurrence, one batch row
    (or, with heads_per_block, one block of heads of a row) at a time, through StreamGate:
    the whole-array gate without holding the whole fp64 reference.  y and fin may live on
    the GPU; the inputs are the host tensors the GPU copy was made from."""
    Bt, L, H, P = (int(s) for s in inp.x.shape)
    hb = heads_per_block or H
    in_dt = DT_NAME[inp.x.dtype]
    gy = StreamGate(in_dt, in_dt, name + " y")
    gf = StreamGate(DT_NAME[fin.dtype], in_dt, name + " final")
    for b in range(Bt):
        for h0 in range(0, H, hb):
            h1 = min(H, h0 + hb)
            yr, fr, _ = oracle.recurrence(**inp.args(), bh=[(b, h) for h in range(h0, h1)])  # [nh, L, P]
            yg = y[b, :, h0:h1].permute(1, 0, 2).to(torch.float64).cpu()
            skip = None
            if inp.D is not None:
                skip = inp.x[b, :, h0:h1].permute(1, 0, 2).to(torch.float64) * \
                    inp.D[h0:h1].to(torch.float64)[:, None, None]
            gy.add(yg, yr, skip)
            gf.add(fin[b, h0:h1].to(torch.float64).cpu(), fr)
            del yr, yg, skip
    return gy.finish(), gf.finish()
