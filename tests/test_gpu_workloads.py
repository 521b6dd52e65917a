"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The oracle evaluates whole sequences for a fixed sample of (batch, head) chains (each
chain is independent), so every token of those chains is compared; the 130M layer is
compared in full.
"""
import pytest
import torch

from gpu_common import check_full, check_sampled, require_gpu, run_gpu, say
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


# "fused" is the form the library picks (relay items here and for the long contexts); the
# chunk tiles' own hop is covered at these sizes too
@pytest.mark.parametrize("impl", ["fused", "fused_hop", "unfused"])
def test_mamba2_130m_full(impl):
    w = WORKLOADS["mamba2_130m_f16"]
    inp = inputs_for(w.name)
    say(w.name, impl)
    y, fin = run_gpu(inp, w.chunk_size, impl)
    check_full(inp, y, fin, w.name + " " + impl)


PAIRS_2P7B = [(0, 0), (7, 79), (3, 17), (5, 40), (1, 63), (6, 5)]


@pytest.mark.parametrize("impl", ["fused", "unfused"])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_mamba2_2p7b_sampled(Q, impl):
    w = WORKLOADS["mamba2_2p7b_bf16"]
    inp = inputs_for(w.name)
    say(w.name, "Q", Q, impl)
    y, fin = run_gpu(inp, Q, impl)
    check_sampled(inp, y, fin, PAIRS_2P7B, "%s Q%d %s" % (w.name, Q, impl))
    del y, fin
    torch.cuda.empty_cache()


@pytest.mark.parametrize("impl", ["fused", "unfused"])
def test_short_g8_sampled(impl):
    w = WORKLOADS["short_g8_bf16"]
    inp = inputs_for(w.name)
    say(w.name, impl)
    y, fin = run_gpu(inp, w.chunk_size, impl)
    check_sampled(inp, y, fin, [(0, 0), (31, 127), (9, 16), (17, 15), (20, 100)], w.name + " " + impl)


@pytest.mark.parametrize("name,impl", [("long_131k_f16", "fused"), ("long_131k_f16", "fused_hop"),
                                       ("long_131k_f16", "unfused"), ("long_262k_f16", "fused"),
                                       ("long_262k_f16", "unfused")])
def test_long_context_sampled(name, impl):
    w = WORKLOADS[name]
    inp = inputs_for(name)
    say(name, impl)
    y, fin = run_gpu(inp, w.chunk_size, impl, state_dtype=torch.float16)
    check_sampled(inp, y, fin, [(0, 0), (0, 33), (0, 79), (0, 50)], name + " " + impl)
    del y, fin
    torch.cuda.empty_cache()


@pytest.mark.parametrize("impl", ["fused", "unfused"])
def test_mamba2_2p7b_fp16_state_sampled(impl):
    """The 2.7B layer with fp16 state storage (the initial state, every inter-chunk state and
    the final state): the relaxed-state point bench.py reports beside the fp32-state headline."""
    import copy
    w = WORKLOADS["mamba2_2p7b_bf16"]
    inp = copy.copy(inputs_for(w.name))
    inp.h0 = inp.h0.to(torch.float16)
    say(w.name, "fp16 state", impl)
    y, fin = run_gpu(inp, w.chunk_size, impl, state_dtype=torch.float16)
    check_sampled(inp, y, fin, PAIRS_2P7B, "%s fp16 state %s" % (w.name, impl))
    del y, fin
    torch.cuda.empty_cache()
