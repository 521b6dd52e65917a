"""Relaxed intermediates ("Mamba-2炸裂升级！…", section "精度与性能的平衡艺术": exact versus
relaxed dtypes): with relaxed = 1 the bmm step stores CB = C B^T of each chunk in the 16-bit
input type instead of fp32.  The result is held to the same parity gate against the fp64
oracle.  Cases cover every way the chunk tile reads CB: into registers for the L bands
(P >= 64 at Q <= 128), as LDS bands (4 heads per tile at Q = 128), straight from memory
(Q = 256); both forms and the relay form; packed input; and the full 2.7B layer, every chain.
"""
import numpy as np
import pytest
import torch

import mamba_ssd_prefill_amd as ssd
import oracle
from gpu_common import DT_NAME, check_all_chains, check_full, f64, fused_form, require_gpu, run_gpu, say
from mamba_ssd_prefill_amd.inputs import WORKLOADS, make_inputs, workload_inputs
from parity import gate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def dev():
    return require_gpu()


CASES = [  # dtype, state, h0, B, L, H, P, N, G, Q
    ("bf16", "f32", True, 2, 5 * 128 + 17, 8, 64, 128, 2, 128),   # L bands from registers
    ("f16", "f16", True, 1, 4 * 128 + 3, 8, 32, 128, 1, 128),    # CB bands in LDS (4 heads per tile)
    ("bf16", "f32", False, 1, 3 * 256 + 100, 4, 64, 128, 1, 256),  # CB straight from memory
    ("f16", "f32", True, 2, 7 * 64 + 1, 8, 64, 64, 4, 64),
    ("bf16", "f32", True, 1, 2 * 128 + 60, 4, 128, 64, 1, 128),
    ("bf16", "f32", True, 1, 600, 8, 16, 32, 2, 128),
]


@pytest.mark.parametrize("impl", ["unfused", "fused_hop", "fused_relay2"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_relaxed_small(case, impl):
    dt, st, h0, B, L, H, P, N, G, Q = case
    say("relaxed", case, impl)
    inp = make_inputs(B, L, H, P, N, G, dtype=dt, state_dtype=st, has_h0=h0, seed=3000 + L + P)
    sd = {"f32": torch.float32, "f16": torch.float16}[st]
    y, fin = run_gpu(inp, Q, impl, state_dtype=sd, relaxed=True)
    r1, r2 = check_full(inp, y, fin, "relaxed %s %s" % (case, impl))
    say("  net normalised err y %.3g final %.3g" % (r1["normalised_err_net"], r2["normalised_err_net"]))


def test_relaxed_packed_input():
    L, Q = 900, 128
    inp = make_inputs(1, L, 8, 64, 128, 2, dtype="bf16", state_dtype="f32", has_h0=True, seed=3100)
    lens = [1, 127, 3, 200, 5, 64, 300]
    seq = np.zeros((1, L), dtype=np.int32)
    t = 0
    for k, n in enumerate(lens):
        seq[0, t:t + n] = k
        t += n
    seq[0, t:] = len(lens)
    seq = torch.from_numpy(seq)
    g = inp.to("cuda:0")
    with fused_form("fused") as name:
        y, fin = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q, impl=name,
                                 seq_idx=seq.to("cuda:0"), relaxed=True)
    torch.cuda.synchronize()
    yr, fr = oracle.recurrence_varlen(**inp.args(), seq_idx=seq)
    skip = f64(inp.D)[None, None, :, None] * f64(inp.x)
    gate(f64(y), yr, "bf16", "bf16", skip=skip, name="relaxed packed y")
    gate(f64(fin), fr, "f32", "bf16", name="relaxed packed final")


@pytest.mark.parametrize("Q", [128, 256])
def test_relaxed_2p7b_full(Q):
    w = WORKLOADS["mamba2_2p7b_bf16"]
    inp = workload_inputs(w)
    say("relaxed 2.7B Q", Q)
    y, fin = run_gpu(inp, Q, "fused", relaxed=True)
    ry, rf = check_all_chains(inp, y, fin, "relaxed 2.7B Q%d" % Q)
    say("  net normalised err y %.3g final %.3g" % (ry["normalised_err_net"], rf["normalised_err_net"]))
    del y, fin
    torch.cuda.empty_cache()
