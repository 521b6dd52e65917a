"""The parity gate must reject plausible kernel mistakes (CPU only).

Each mutant below is the chunked algorithm with one mistake planted, evaluated in
fp64 on the CPU and rounded to the output dtypes the GPU stores.  The gate in
tests/parity.py has to reject every one of them against the oracle, while the
same evaluation without a mistake passes.  Inputs follow the workload recipe at
a reduced size (several chunks, nonzero and zero initial state).
"""
import numpy as np
import pytest
import torch

from mamba_ssd_prefill_amd.inputs import make_inputs
from parity import ParityError, gate

MUTANTS = [
    "none",
    "skip_state_passing",   # every chunk starts from the initial state
    "drop_D",               # skip term missing
    "strict_mask",          # j < i instead of j <= i on the diagonal block
    "leaky_mask",           # includes token i+1
    "strided_group_map",    # g = h % G instead of h // (H/G)
    "decay_sign",           # exp(Acs_j - Acs_i) on the diagonal block
    "no_dt_in_state",       # chunk_state drops the dt weight
    "stale_final_state",    # final state misses the last chunk's hop
    "no_state_decay",       # state passing forgets exp(Acs_last)
    "off_term_undecayed",   # chunk_scan forgets exp(Acs_i) on C S_c
    "cb_transposed",        # uses B C^T instead of C B^T
]


def f64(t):
    return None if t is None else t.detach().to(torch.float64).numpy()


def chunked_numpy(inp, Q, mutant="none"):
    x, dtr, A, Bm, Cm = f64(inp.x), f64(inp.dt), f64(inp.A), f64(inp.B), f64(inp.C)
    D, bias, h0 = f64(inp.D), f64(inp.dt_bias), f64(inp.h0)
    Bt, L, H, P = x.shape
    G, N = Bm.shape[2:]
    hpg = H // G
    nc = -(-L // Q)
    d = np.logaddexp(0.0, dtr + bias[None, None, :])
    y = np.zeros_like(x)
    fin = np.zeros((Bt, H, P, N))
    for b in range(Bt):
        for h in range(H):
            g = (h % G) if mutant == "strided_group_map" else h // hpg
            S = h0[b, h].copy() if h0 is not None else np.zeros((P, N))
            S_prev = S.copy()
            for c in range(nc):
                t0, t1 = c * Q, min(L, (c + 1) * Q)
                dc = d[b, t0:t1, h]
                acs = np.cumsum(dc * A[h])
                Xc, Bc, Cc = x[b, t0:t1, h], Bm[b, t0:t1, g], Cm[b, t0:t1, g]
                CB = Bc @ Cc.T if mutant == "cb_transposed" else Cc @ Bc.T
                n = t1 - t0
                ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
                mask = jj < ii if mutant == "strict_mask" else (jj <= ii + 1 if mutant == "leaky_mask" else jj <= ii)
                seg = acs[None, :] - acs[:, None] if mutant == "decay_sign" else acs[:, None] - acs[None, :]
                Lm = np.where(mask, CB * np.exp(np.where(mask, seg, 0.0)) * dc[None, :], 0.0)
                S_in = h0[b, h] if (mutant == "skip_state_passing" and h0 is not None) else \
                    (np.zeros((P, N)) if mutant == "skip_state_passing" else S)
                off = Cc @ S_in.T
                if mutant != "off_term_undecayed":
                    off = np.exp(acs)[:, None] * off
                yc = off + Lm @ Xc
                if mutant != "drop_D":
                    yc = yc + D[h] * Xc
                y[b, t0:t1, h] = yc
                w = np.exp(acs[-1] - acs) * (1.0 if mutant == "no_dt_in_state" else dc)
                s_loc = (Xc * w[:, None]).T @ Bc
                S_prev = S
                decay = 1.0 if mutant == "no_state_decay" else np.exp(acs[-1])
                S = decay * S + s_loc
            fin[b, h] = S_prev if mutant == "stale_final_state" else S
    return y, fin


def _round(a, dtype):
    t = torch.from_numpy(a).to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype])
    return t.to(torch.float64).numpy()


CASES = [
    dict(name="bf16_h0", dtype="bf16", state="f32", h0=True, seed=21),
    dict(name="bf16_zero_h0", dtype="bf16", state="f32", h0=False, seed=22),
    dict(name="f16_f16state", dtype="f16", state="f16", h0=True, seed=23),
    dict(name="f32_tiny", dtype="f32", state="f32", h0=False, seed=24),
]


@pytest.fixture(scope="module")
def cases(oracle_mod):
    out = {}
    for cs in CASES:
        inp = make_inputs(1, 320, 4, 16, 32, 2, dtype=cs["dtype"], state_dtype=cs["state"],
                          has_h0=cs["h0"], seed=cs["seed"])
        y, fin = oracle_mod.recurrence_full(**inp.args())
        out[cs["name"]] = (cs, inp, y, fin)
    return out


@pytest.mark.parametrize("case", [c["name"] for c in CASES])
@pytest.mark.parametrize("mutant", MUTANTS)
def test_gate_rejects_planted_mistakes(cases, case, mutant):
    cs, inp, yref, finref = cases[case]
    Q = 64
    y, fin = chunked_numpy(inp, Q, mutant)
    y = _round(y, cs["dtype"])
    fin = _round(fin, cs["state"])
    skip = f64(inp.D)[None, None, :, None] * f64(inp.x)

    def passes():
        try:
            gate(y, yref, cs["dtype"], cs["dtype"], skip=skip, name="y")
            gate(fin, finref, cs["state"], cs["dtype"], name="final")
            return True
        except ParityError:
            return False

    if mutant == "none":
        assert passes()
    else:
        assert not passes(), "gate accepted mutant %s" % mutant
