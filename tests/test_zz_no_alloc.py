"""ssd_prefill_noalloc (the library's static scratch as the workspace) through the C ABI.

Its outputs must equal ssd_prefill's with a caller workspace, element for element, and pass the
parity gate against the fp64 oracle, on two calls in a row on one GPU, the second with a smaller
problem (the scratch keeps the first call's contents).  (The refusal of a problem larger than the
scratch is a CPU test in test_abi.py.)
"""
import pytest
import torch

import mamba_ssd_prefill_amd as ssd
from gpu_common import check_full, fused_form, require_gpu, say
from mamba_ssd_prefill_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def dev():
    return require_gpu()


def both(inp, Q, impl):
    g = inp.to("cuda:0")
    with fused_form(impl) as name:
        y0, f0 = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q, impl=name)
        y1 = torch.full_like(y0, float("nan"))
        f1 = torch.full_like(f0, float("nan"))
        ssd.ssd_prefill_noalloc(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q, impl=name,
                                y=y1, final_state=f1)
    torch.cuda.synchronize()
    return y0, f0, y1, f1


@pytest.mark.parametrize("impl", ["fused", "fused_hop", "fused_relay2", "unfused"])
def test_noalloc_matches_prefill_twice_second_smaller(impl):
    first = make_inputs(2, 1000, 8, 64, 128, 2, dtype="bf16", state_dtype="f32", has_h0=True, seed=71)
    second = make_inputs(1, 300, 4, 64, 128, 1, dtype="bf16", state_dtype="f32", has_h0=False, seed=72)
    for k, (inp, Q) in enumerate(((first, 128), (second, 64))):
        say("noalloc call", k, impl)
        y0, f0, y1, f1 = both(inp, Q, impl)
        assert torch.equal(y0, y1) and torch.equal(f0, f1)
        check_full(inp, y1, f1, "noalloc %d %s" % (k, impl))

