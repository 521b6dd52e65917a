"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Every element of y and of the final state of every (batch, head) chain is compared with
the fp64 recurrence: the oracle runs one batch row (or, for the single-row long contexts,
one block of 16 heads) at a time and StreamGate applies the parity gate to the whole
array block by block.  Each config runs in the default fused form and the unfused form,
the 2.7B layer at every chunk size of the bench sweep, and the relay-form shapes also in
the chunk tiles' own hop form.
"""
import copy

import pytest
import torch

from gpu_common import check_all_chains, require_gpu, run_gpu, say
from mamba_ssd_prefill_amd.inputs import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def dev():
    return require_gpu()


_cache = {}


def inputs_for(name):
    if name not in _cache:
        _cache.clear()
        say("generating", name)
        _cache[name] = workload_inputs(WORKLOADS[name])
    return _cache[name]


def _run_and_check(inp, Q, impl, label, state_dtype=None, heads_per_block=0):
    say(label)
    y, fin = run_gpu(inp, Q, impl, state_dtype=state_dtype)
    ry, rf = check_all_chains(inp, y, fin, label, heads_per_block)
    say("  %s: y %d elements, net normalised err %.3g; final net normalised err %.3g"
        % (label, ry["elements"], ry["normalised_err_net"], rf["normalised_err_net"]))
    del y, fin
    torch.cuda.empty_cache()


# "fused" is the form the library picks (relay items here and for the long contexts); the
# chunk tiles' own hop is covered at these sizes too
@pytest.mark.parametrize("impl", ["fused", "fused_hop", "unfused"])
def test_mamba2_130m_full(impl):
    w = WORKLOADS["mamba2_130m_f16"]
    _run_and_check(inputs_for(w.name), w.chunk_size, impl, "%s %s" % (w.name, impl))


@pytest.mark.parametrize("impl", ["fused", "unfused"])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_mamba2_2p7b_full(Q, impl):
    w = WORKLOADS["mamba2_2p7b_bf16"]
    _run_and_check(inputs_for(w.name), Q, impl, "%s Q%d %s" % (w.name, Q, impl))


def test_mamba2_2p7b_full_no_D():
    """The full 2.7B layer with D = 0: y is the SSM term alone, so the contract tolerance itself
    (not only the normalised check) sees every error of the scan."""
    w = WORKLOADS["mamba2_2p7b_bf16"]
    inp = copy.copy(inputs_for(w.name))
    inp.D = None
    _run_and_check(inp, w.chunk_size, "fused", "%s D=0 fused" % w.name)


@pytest.mark.parametrize("impl", ["fused", "unfused"])
def test_short_g8_full(impl):
    w = WORKLOADS["short_g8_bf16"]
    _run_and_check(inputs_for(w.name), w.chunk_size, impl, "%s %s" % (w.name, impl))


@pytest.mark.parametrize("name,impl", [("long_131k_f16", "fused"), ("long_131k_f16", "fused_hop"),
                                       ("long_131k_f16", "unfused"), ("long_262k_f16", "fused"),
                                       ("long_262k_f16", "unfused")])
def test_long_context_full(name, impl):
    w = WORKLOADS[name]
    _run_and_check(inputs_for(name), w.chunk_size, impl, "%s %s" % (name, impl), state_dtype=torch.float16,
                   heads_per_block=16)


@pytest.mark.parametrize("impl", ["fused", "unfused"])
def test_mamba2_2p7b_fp16_state_full(impl):
    """The 2.7B layer with fp16 state storage (the initial state, every inter-chunk state and
    the final state): the relaxed-state point bench.py reports beside the fp32-state headline."""
    w = WORKLOADS["mamba2_2p7b_bf16"]
    inp = copy.copy(inputs_for(w.name))
    inp.h0 = inp.h0.to(torch.float16)
    _run_and_check(inp, w.chunk_size, impl, "%s fp16 state %s" % (w.name, impl), state_dtype=torch.float16)
