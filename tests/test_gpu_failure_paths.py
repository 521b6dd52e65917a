"""The fused kernel's failure reporting and its relay-admission fallback, forced from the host.

Every case ends with every kernel exiting normally:
* a tiny MAMBA_SSD_SPIN_LIMIT makes the kernel's own bounded waits give up: the device status
  word must read SSD_ERR_SYNC_TIMEOUT, and the next call (default limit) must be correct and
  read SSD_OK;
* MAMBA_SSD_GRID_LIMIT=1 launches one workgroup, which serves its own XCD's partition and
  leaves the others unserved: SSD_ERR_SCHEDULE (no wait crosses partitions, so nothing hangs);
* MAMBA_SSD_RELAY_ADMIT=0 makes every partition of a relay-form launch decide that its chunk
  tiles pass the state themselves: the results must still match the oracle;
* a 256-token-chunk shape with about 100 chains, where the relay items would not fit the one
  workgroup per CU that tile's LDS allows, must be correct in the form the library picks.
"""
import pytest
import torch

import mamba_ssd_prefill_amd as ssd
from gpu_common import DT_NAME, check_full, fused_form, require_gpu, run_gpu, say
from mamba_ssd_prefill_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

SSD_ERR_SYNC_TIMEOUT, SSD_ERR_SCHEDULE = 7, 9


@pytest.fixture(scope="module", autouse=True)
def dev():
    return require_gpu()


def run_status(inp, Q, impl):
    """One ssd_prefill; returns (y, final_state, device status) without asserting the status."""
    with fused_form(impl) as name:
        g = inp.to("cuda:0")
        Bt, L, H, P = g.x.shape
        G, N = g.B.shape[2], g.B.shape[3]
        sd = g.h0.dtype if g.h0 is not None else torch.float32
        prm = ssd.make_params(Bt, L, H, P, N, G, Q, DT_NAME[g.x.dtype], DT_NAME[sd], True, name)
        ws = ssd.alloc_workspace(prm, g.x.device)
        y, fin = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q, impl=name,
                                 workspace=ws)
        torch.cuda.synchronize()
        return y, fin, ssd.check_device_status(prm, ws)


@pytest.mark.parametrize("impl", ["fused_hop", "fused_relay2"])
def test_spin_limit_gives_sync_timeout_then_recovers(impl, monkeypatch):
    # one chain of 64 chunks: chunk tile c waits for c earlier hand-offs, far beyond 32 polls
    inp = make_inputs(1, 64 * 128, 2, 64, 128, 1, dtype="bf16", has_h0=True, seed=91)
    monkeypatch.setenv("MAMBA_SSD_SPIN_LIMIT", "1")
    say("spin limit 1", impl)
    _, _, status = run_status(inp, 128, impl)
    assert status == SSD_ERR_SYNC_TIMEOUT
    monkeypatch.delenv("MAMBA_SSD_SPIN_LIMIT")
    y, fin, status = run_status(inp, 128, impl)
    assert status == 0
    check_full(inp, y, fin, "after timeout " + impl)


@pytest.mark.parametrize("impl", ["fused_hop", "fused_relay2"])
def test_unserved_partition_gives_schedule_error(impl, monkeypatch):
    if torch.cuda.get_device_properties(0).multi_processor_count < 16:
        pytest.skip("needs a device with several XCDs")
    inp = make_inputs(4, 600, 8, 64, 128, 2, dtype="bf16", has_h0=True, seed=92)
    monkeypatch.setenv("MAMBA_SSD_GRID_LIMIT", "1")
    say("grid limit 1", impl)
    _, _, status = run_status(inp, 128, impl)
    assert status == SSD_ERR_SCHEDULE
    monkeypatch.delenv("MAMBA_SSD_GRID_LIMIT")
    y, fin, status = run_status(inp, 128, impl)
    assert status == 0
    check_full(inp, y, fin, "after schedule error " + impl)


@pytest.mark.parametrize("has_h0", [True, False])
@pytest.mark.parametrize("L", [5 * 128 + 9, 6 * 128])  # odd and even chunk counts
@pytest.mark.parametrize("case", [("bf16", 64, 128, 128), ("f16", 32, 64, 64), ("f32", 16, 32, 64)],
                         ids=["bf16", "f16", "f32"])
def test_relay_admission_refused_falls_back_to_hop(case, L, has_h0, monkeypatch):
    dt, P, N, Q = case
    inp = make_inputs(2, L, 8, P, N, 2, dtype=dt, has_h0=has_h0, seed=93 + L)
    monkeypatch.setenv("MAMBA_SSD_RELAY_ADMIT", "0")
    say("relay refused", case, L, has_h0)
    y, fin = run_gpu(inp, Q, "fused_relay2")
    check_full(inp, y, fin, "relay refused %s" % (case,))


@pytest.mark.parametrize("impl", ["fused", "fused_relay2", "fused_relay4", "unfused"])
def test_q256_about_100_chains(impl):
    inp = make_inputs(1, 3 * 256 + 40, 200, 64, 128, 1, dtype="bf16", has_h0=True, seed=94)
    say("Q256 100 chains", impl)
    y, fin = run_gpu(inp, 256, impl)
    check_full(inp, y, fin, "Q256 100 chains " + impl)
