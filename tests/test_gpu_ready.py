"""One workspace reused across fused calls with SSD_FLAG_WORKSPACE_READY.

The final-state copy of every fused call resets the workspace's sync words for the next call,
so a flagged call without an initial state skips the launch that would reset them.  Checked:
* runs of flagged calls (new inputs each time, the workspace first filled with 0xFF bytes)
  match the oracle and are bit-identical to calls on a fresh workspace, in the hop form and
  both relay forms, with and without an initial state, and for packed input;
* a flagged call whose previous call on the workspace had other parameters resets as usual;
* after a call whose waits gave up, flagged calls still compute correctly and keep reporting
  SSD_ERR_SYNC_TIMEOUT; the next call without the flag clears it.
"""
import pytest
import torch

import mamba_ssd_prefill_amd as ssd
from gpu_common import DT_NAME, check_full, fused_form, require_gpu, say
from mamba_ssd_prefill_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

SSD_ERR_SYNC_TIMEOUT = 7


@pytest.fixture(scope="module", autouse=True)
def dev():
    return require_gpu()


def params(inp, Q, name):
    Bt, L, H, P = inp.x.shape
    G, N = inp.B.shape[2], inp.B.shape[3]
    sd = inp.h0.dtype if inp.h0 is not None else torch.float32
    return ssd.make_params(Bt, L, H, P, N, G, Q, DT_NAME[inp.x.dtype], DT_NAME[sd], True, name)


def call(inp, Q, name, ws, ready, seq_idx=None):
    g = inp.to("cuda:0")
    y, fin = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q, impl=name, workspace=ws,
                             workspace_ready=ready, seq_idx=seq_idx)
    torch.cuda.synchronize()
    return y, fin


def dirty_workspace(prm):
    ws = ssd.alloc_workspace(prm, "cuda:0")
    ws.fill_(255)
    return ws


@pytest.mark.parametrize("impl", ["fused_hop", "fused_relay2", "fused_relay4"])
@pytest.mark.parametrize("has_h0", [False, True])
def test_flagged_calls_match_fresh_calls(impl, has_h0):
    inps = [make_inputs(2, 1000, 8, 64, 128, 2, dtype="bf16", has_h0=has_h0, seed=400 + i) for i in range(3)]
    with fused_form(impl) as name:
        prm = params(inps[0], 128, name)
        ws = dirty_workspace(prm)
        for i, inp in enumerate(inps):
            say("ready", impl, "h0" if has_h0 else "no h0", "call", i)
            y, fin = call(inp, 128, name, ws, ready=i > 0)
            assert ssd.check_device_status(prm, ws) == 0
            check_full(inp, y, fin, "ready %s call %d" % (impl, i))
            y2, fin2 = call(inp, 128, name, dirty_workspace(prm), ready=False)
            assert torch.equal(y, y2) and torch.equal(fin, fin2)


def test_flagged_packed_input():
    inps = [make_inputs(1, 2000, 8, 64, 128, 1, dtype="f16", has_h0=False, seed=410 + i) for i in range(2)]
    seq = torch.zeros(1, 2000, dtype=torch.int32)
    for s in (300, 301, 900, 1500):
        seq[0, s:] += 1
    seq = seq.to("cuda:0")
    prm = params(inps[0], 128, "fused")
    ws = dirty_workspace(prm)
    outs = [call(inp, 128, "fused", ws, ready=i > 0, seq_idx=seq) for i, inp in enumerate(inps)]
    for (y, fin), inp in zip(outs, inps):
        y2, fin2 = call(inp, 128, "fused", dirty_workspace(prm), ready=False, seq_idx=seq)
        assert torch.equal(y, y2) and torch.equal(fin, fin2)
    assert ssd.check_device_status(prm, ws) == 0


def test_flag_after_other_parameters_resets():
    big = make_inputs(1, 1024, 8, 64, 128, 1, dtype="bf16", has_h0=False, seed=420)
    small = make_inputs(1, 300, 8, 64, 128, 1, dtype="bf16", has_h0=False, seed=421)
    ws = dirty_workspace(params(big, 128, "fused"))
    for i, inp in enumerate((big, small, big, big)):
        say("ready across shapes, call", i)
        y, fin = call(inp, 128, "fused", ws, ready=i > 0)
        check_full(inp, y, fin, "ready across shapes %d" % i)
        assert ssd.check_device_status(params(inp, 128, "fused"), ws) == 0


@pytest.mark.parametrize("impl", ["fused_hop", "fused_relay2"])
def test_status_stays_until_a_call_without_the_flag(impl, monkeypatch):
    inp = make_inputs(1, 64 * 128, 2, 64, 128, 1, dtype="bf16", has_h0=False, seed=430)
    with fused_form(impl) as name:
        prm = params(inp, 128, name)
        ws = dirty_workspace(prm)
        monkeypatch.setenv("MAMBA_SSD_SPIN_LIMIT", "1")
        say("ready after timeout", impl)
        call(inp, 128, name, ws, ready=False)
        assert ssd.check_device_status(prm, ws) == SSD_ERR_SYNC_TIMEOUT
        monkeypatch.delenv("MAMBA_SSD_SPIN_LIMIT")
        y, fin = call(inp, 128, name, ws, ready=True)
        check_full(inp, y, fin, "ready after timeout " + impl)
        assert ssd.check_device_status(prm, ws) == SSD_ERR_SYNC_TIMEOUT
        y, fin = call(inp, 128, name, ws, ready=False)
        check_full(inp, y, fin, "reset after timeout " + impl)
        assert ssd.check_device_status(prm, ws) == 0
