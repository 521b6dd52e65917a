"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Sizes here finish in seconds on the oracle while spanning several chunk tiles and a
ragged last chunk; tests/test_gpu_workloads.py covers the full workload sizes.
"""
import zlib

import numpy as np
import pytest
import torch

import mamba_ssd_prefill_amd as ssd
import oracle
from gpu_common import check_full, f64, require_gpu, run_gpu, say
from mamba_ssd_prefill_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from parity import gate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def dev():
    return require_gpu()


# the fused form both with the chunk tiles' own state hop and with relay items (2 and 4
# relay waves per chain part)
IMPLS = ["unfused", "fused_hop", "fused_relay2", "fused_relay4"]


@pytest.mark.parametrize("impl", IMPLS)
def test_tiny_f32_workload(impl):
    w = WORKLOADS["tiny_f32"]
    say("tiny_f32", impl)
    inp = workload_inputs(w)
    y, fin = run_gpu(inp, w.chunk_size, impl)
    check_full(inp, y, fin, "tiny_f32 " + impl)


CASES = [
    # dtype, state dtype, h0, B, L, H, P, N, G, Q
    ("bf16", "f32", True, 2, 1000, 8, 64, 128, 2, 128),
    ("bf16", "f32", False, 1, 777, 8, 64, 128, 1, 64),
    ("f16", "f32", False, 2, 640, 6, 64, 128, 1, 128),
    ("f16", "f16", True, 1, 1100, 8, 64, 128, 1, 128),
    ("bf16", "f32", True, 1, 900, 4, 64, 128, 1, 256),
    ("f16", "f32", True, 2, 700, 4, 64, 64, 2, 256),
    ("f32", "f32", True, 1, 300, 4, 64, 128, 1, 128),
    ("bf16", "f32", True, 2, 333, 8, 32, 64, 4, 64),
    ("bf16", "f32", True, 1, 400, 6, 16, 32, 3, 128),
    ("bf16", "f32", True, 1, 500, 2, 128, 128, 1, 128),
    ("f16", "f32", True, 3, 200, 12, 64, 64, 12, 64),   # G = H
    ("bf16", "bf16", True, 1, 260, 4, 64, 128, 1, 128),
    ("f32", "f32", False, 1, 256, 4, 16, 16, 1, 64),
    # y leaves through LDS in whole token rows when every head of a tile is valid: four heads
    # per tile at P = 32; and 3 heads per group at P = 64, where one tile of each group holds a
    # single head and stores y directly, in the same launch
    ("bf16", "f32", True, 1, 300, 8, 32, 128, 1, 128),
    ("bf16", "f32", True, 2, 300, 6, 64, 128, 2, 128),
    # 41 chunks: wraps the relay form's 10-slot chunk-state ring and 6-slot operand ring several times
    ("bf16", "f32", True, 1, 40 * 128 + 7, 4, 64, 128, 1, 128),
    ("f16", "f16", True, 1, 40 * 64 + 33, 2, 64, 64, 1, 64),
]


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_parity_small(impl, case):
    dt, st, h0, B, L, H, P, N, G, Q = case
    say("case", case, impl)
    inp = make_inputs(B, L, H, P, N, G, dtype=dt, state_dtype=st, has_h0=h0, seed=zlib.crc32(repr(case).encode()) % 100000)
    sd = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[st]
    y, fin = run_gpu(inp, Q, impl, state_dtype=sd)
    check_full(inp, y, fin, str(case) + " " + impl)


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("L", [1, 5, 63, 64, 65, 127, 128, 129])
def test_short_and_boundary_lengths(impl, L):
    say("length", L, impl)
    inp = make_inputs(2, L, 4, 64, 128, 1, dtype="bf16", has_h0=True, seed=L)
    y, fin = run_gpu(inp, 64, impl)
    check_full(inp, y, fin, "L=%d" % L)


@pytest.mark.parametrize("impl", IMPLS)
def test_no_D_no_bias_no_softplus(impl):
    say("no D / bias / softplus", impl)
    inp = make_inputs(1, 300, 4, 64, 128, 1, dtype="bf16", has_h0=True, seed=5, with_D=False)
    inp.dt_bias = None
    inp.dt = (0.05 * inp.dt.float().abs()).to(torch.bfloat16)
    inp.dt_softplus = False
    y, fin = run_gpu(inp, 128, impl)
    check_full(inp, y, fin, "noD")


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_negative_steps(impl, dtype):
    """dt_softplus = 0 with steps of either sign (dt = dt_raw, no bias): a negative step makes
    dt * A > 0, so the in-chunk decay sums rise and fall; the recurrence (and the oracle) grow
    the state there.  Every decay must stay finite and exact, the diagonal block included."""
    say("negative steps", dtype, impl)
    inp = make_inputs(2, 333, 4, 64, 128, 1, dtype=dtype, has_h0=True, seed=55)
    inp.dt_bias = None
    inp.dt = (0.02 * inp.dt.float()).to(inp.x.dtype)
    inp.dt_softplus = False
    assert bool((inp.dt.float() < 0).any()) and bool((inp.dt.float() > 0).any())
    y, fin = run_gpu(inp, 64 if dtype == "f32" else 128, impl)
    check_full(inp, y, fin, "negative dt %s" % dtype)


@pytest.mark.parametrize("impl", IMPLS)
def test_linear_attention_case(impl):
    """A = 0, dt = 1: causal linear attention (no decay)."""
    say("linear attention", impl)
    inp = make_inputs(1, 256, 4, 64, 128, 1, dtype="f32", has_h0=False, seed=6)
    inp.A = torch.zeros_like(inp.A)
    inp.dt = torch.ones_like(inp.dt)
    inp.dt_bias = torch.zeros_like(inp.dt_bias)
    inp.dt_softplus = False
    inp.B = inp.B * 0.25
    y, fin = run_gpu(inp, 64, impl)
    X, Bm, Cm = f64(inp.x), f64(inp.B), f64(inp.C)
    M = np.tril(Cm[0, :, 0] @ Bm[0, :, 0].T)
    for h in range(4):
        ref = M @ X[0, :, h] + float(inp.D[h]) * X[0, :, h]
        assert np.max(np.abs(f64(y)[0, :, h] - ref)) < 1e-4 * max(1.0, np.max(np.abs(ref)))
    check_full(inp, y, fin, "linattn")


@pytest.mark.parametrize("impl", IMPLS)
def test_zero_input_exact_zero(impl):
    inp = make_inputs(1, 200, 4, 64, 128, 1, dtype="bf16", has_h0=False, seed=7)
    inp.x = torch.zeros_like(inp.x)
    y, fin = run_gpu(inp, 64, impl)
    assert torch.count_nonzero(y).item() == 0 and torch.count_nonzero(fin).item() == 0


@pytest.mark.parametrize("impl", IMPLS)
def test_zero_step_keeps_state(impl):
    inp = make_inputs(1, 200, 4, 64, 128, 1, dtype="bf16", has_h0=True, seed=8)
    inp.dt = torch.zeros_like(inp.dt)
    inp.dt_bias = torch.zeros_like(inp.dt_bias)
    inp.dt_softplus = False
    y, fin = run_gpu(inp, 64, impl)
    assert torch.equal(fin.cpu(), inp.h0)
    check_full(inp, y, fin, "dt0")


@pytest.mark.parametrize("form", ["fused_hop", "fused_relay2", "fused_relay4"])
def test_fused_is_deterministic_and_matches_unfused(form):
    inp = make_inputs(2, 1000, 8, 64, 128, 2, dtype="bf16", has_h0=True, seed=9)
    y1, f1 = run_gpu(inp, 128, form)
    y2, f2 = run_gpu(inp, 128, form)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    yu, fu = run_gpu(inp, 128, "unfused")
    # both evaluate the same arithmetic per tile; only the state chain's rounding differs
    gate(f64(y1), f64(yu), "bf16", "bf16", name="fused vs unfused y")
    gate(f64(f1), f64(fu), "f32", "bf16", name="fused vs unfused final")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("group", [1, 3, 7])
def test_claim_groups_change_nothing(group, dtype, monkeypatch):
    """Chains claimed in groups (MAMBA_SSD_CHAIN_GROUP; chosen automatically for many short
    chains) give the same bits as one group: only the order of the claims changes."""
    # 4 batch rows x 2 groups x 16 heads: 32 two-head chains (4 per partition) at 16 bits, 8 chunks
    inp = make_inputs(4, 1000, 16, 64, 128, 2, dtype=dtype, has_h0=True, seed=12)
    say("claim groups", group, dtype)
    y0, f0 = run_gpu(inp, 128, "fused_hop")
    monkeypatch.setenv("MAMBA_SSD_CHAIN_GROUP", str(group))
    y1, f1 = run_gpu(inp, 128, "fused_hop")
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    check_full(inp, y1, f1, "claim groups %d" % group)


def test_workspace_reuse_across_shapes():
    """A workspace sized for a larger call is reused for a smaller one (flags reset)."""
    big = make_inputs(1, 1024, 8, 64, 128, 1, dtype="bf16", has_h0=True, seed=10)
    small = make_inputs(1, 300, 8, 64, 128, 1, dtype="bf16", has_h0=True, seed=11)
    prm = ssd.make_params(1, 1024, 8, 64, 128, 1, 128, "bf16", "f32", True, "fused")
    ws = torch.empty(ssd.workspace_size(prm), dtype=torch.uint8, device="cuda:0")
    for inp in (big, small, big):
        g = inp.to("cuda:0")
        y, fin = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=128, workspace=ws)
        torch.cuda.synchronize()
        check_full(inp, y, fin, "reuse")
    assert ssd.check_device_status(prm, ws) == 0


# ---- per-step parity of the unfused form -------------------------------------------------------
@pytest.mark.parametrize("dtype,Q,L", [("bf16", 128, 1000), ("f32", 64, 300), ("f16", 256, 600)])
def test_unfused_steps_match_chunked_oracle(dtype, Q, L):
    say("steps", dtype, Q, L)
    Bt, H, P, N, G = 2, 8, 64, 128, 2
    inp = make_inputs(Bt, L, H, P, N, G, dtype=dtype, has_h0=True, seed=12)
    ref = oracle.chunked(**inp.args(), chunk_size=Q)
    prm = ssd.make_params(Bt, L, H, P, N, G, Q, dtype, "f32", True, "unfused")
    lay = ssd.workspace_layout(prm)
    g = inp.to("cuda:0")
    ws = torch.zeros(lay.total_bytes, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(g.x)
    fin = torch.empty(Bt, H, P, N, device="cuda:0")
    nc = lay.nchunks

    def region(off, nbytes, shape):
        return ws[off:off + nbytes].view(torch.float32).reshape(shape).cpu().double().numpy()

    ssd.step_chunk_cumsum(prm, g.dt, g.A, g.dt_bias, ws)
    torch.cuda.synchronize()
    dt_g = region(lay.dt_offset, lay.dt_bytes, (Bt, nc, H, Q))
    acs_g = region(lay.acs_offset, lay.acs_bytes, (Bt, nc, H, Q))
    assert np.all(np.abs(dt_g - ref["dt"]) <= 1e-6 + 1e-5 * np.abs(ref["dt"]))
    scale = np.max(np.abs(ref["acs"]))
    assert np.max(np.abs(acs_g - ref["acs"])) <= 1e-6 * Q * max(scale, 1.0)

    ssd.step_bmm(prm, g.B, g.C, ws)
    torch.cuda.synchronize()
    cb_g = region(lay.cb_offset, lay.cb_bytes, (Bt, nc, G, Q, Q))
    tril = np.tril(np.ones((Q, Q), dtype=bool))
    d = np.abs(cb_g - ref["cb"])[..., tril]
    assert np.max(d) <= 1e-5 + 1e-4 * np.max(np.abs(ref["cb"]))

    ssd.step_chunk_state(prm, g.x, g.B, ws)
    torch.cuda.synchronize()
    s_g = region(lay.s_offset, lay.s_bytes, (Bt, nc, H, P, N))
    tau = 1e-5 if dtype == "f32" else 1e-2
    assert np.max(np.abs(s_g - ref["s"])) <= tau * np.max(np.abs(ref["s"]))

    ssd.step_state_passing(prm, g.h0, fin, ws)
    torch.cuda.synchronize()
    st_g = region(lay.states_offset, lay.states_bytes, (Bt, nc + 1, H, P, N))
    assert np.max(np.abs(st_g - ref["states"])) <= tau * np.max(np.abs(ref["states"]))
    assert np.max(np.abs(f64(fin) - ref["final"])) <= tau * np.max(np.abs(ref["final"]))

    ssd.step_chunk_scan(prm, g.x, g.C, g.D, y, ws)
    torch.cuda.synchronize()
    in_dt = dtype
    gate(f64(y), ref["y"], in_dt, in_dt, skip=f64(inp.D)[None, None, :, None] * f64(inp.x), name="steps y")
