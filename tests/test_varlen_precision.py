"""Packed-input precision of the in-chunk decays (CPU, float32 emulation of the cumsum step).

The chunk_cumsum step forms acs, the inclusive in-chunk sum of dt * A, in fp32: each lane adds
its Q / 64 consecutive tokens, then a wave-wide (Hillis-Steele) scan adds the lane totals.
Every decay the later steps use is exp(acs_i - acs_j) for two tokens of one sequence.  Packed
sequences are told apart by masks on per-chunk start counts ("Mamba-2炸裂升级！…", section
"与vLLM的深度融合": masking by sequence index), so acs is the same array as for unpacked input
and a chunk with 31 sequence starts keeps the precision of one with none.  The emulation also
shows what an offset encoding (a large negative log-decay added at every start) would cost:
its |acs| grows with every start and its rounding lands in every later decay of the chunk.
"""
import numpy as np
import pytest

from mamba_ssd_prefill_amd.inputs import make_inputs


def wave_scan_acs(dA, Q):
    """acs as the cumsum step forms it, in float32 (dA: float32 [Q])."""
    V = Q // 64
    run = np.zeros(Q, dtype=np.float32)
    tot = np.zeros(64, dtype=np.float32)
    for lane in range(64):
        s = np.float32(0)
        for k in range(V):
            s = np.float32(s + dA[lane * V + k])
            run[lane * V + k] = s
        tot[lane] = s
    incl = tot.copy()
    off = 1
    while off < 64:
        prev = incl.copy()
        for lane in range(off, 64):
            incl[lane] = np.float32(prev[lane] + prev[lane - off])
        off *= 2
    excl = (incl - tot).astype(np.float32)
    return np.array([np.float32(excl[i // V] + run[i]) for i in range(Q)], dtype=np.float32)


def worst_decay_error(dA, starts, Q, offset=None):
    """Largest relative error of exp(acs_i - acs_j) over token pairs j < i of one sequence,
    against the exact decay of the same float32 steps."""
    seg = np.cumsum(starts)                        # sequence starts among tokens 0..i
    dAx = dA.copy()
    if offset is not None:
        dAx = (dAx + np.float32(offset) * starts).astype(np.float32)
    acs = wave_scan_acs(dAx, Q).astype(np.float64)
    exact = np.cumsum(dA.astype(np.float64))
    worst = 0.0
    for i in range(Q):
        for j in range(i):
            if seg[i] != seg[j]:
                continue
            got = np.exp(acs[i] - acs[j])
            ref = np.exp(exact[i] - exact[j])
            worst = max(worst, abs(got - ref) / ref)
    return worst


def chunk_steps(Q, seed):
    inp = make_inputs(1, Q, 1, 16, 16, 1, dtype="f32", seed=seed)
    z = inp.dt.double()[0, :, 0] + float(inp.dt_bias[0])
    dt = np.logaddexp(0.0, z.numpy()).astype(np.float32)
    return (dt * np.float32(inp.A[0])).astype(np.float32)


@pytest.mark.parametrize("Q", [64, 128])
def test_masked_decays_keep_fp32_precision(Q):
    dA = chunk_steps(Q, 321 + Q)
    none = np.zeros(Q, dtype=np.int64)
    many = np.zeros(Q, dtype=np.int64)
    many[1:32] = 1                                  # 31 one-token sequences, then one long one
    base = worst_decay_error(dA, none, Q)
    masked = worst_decay_error(dA, many, Q)
    assert masked <= base + 1e-12                   # the same sums: nothing lost to packing
    assert base < 1e-6                              # fp32 rounding of in-chunk sums (~1e-7 here)


@pytest.mark.parametrize("Q", [64, 128])
def test_offset_encoding_would_lose_precision(Q):
    """The emulation discriminates: an offset of -128 per start degrades the decays of the
    chunk's later sequences by an order of magnitude."""
    dA = chunk_steps(Q, 321 + Q)
    many = np.zeros(Q, dtype=np.int64)
    many[1:32] = 1
    base = worst_decay_error(dA, np.zeros(Q, dtype=np.int64), Q)
    assert worst_decay_error(dA, many, Q, offset=-128.0) > 10 * base
