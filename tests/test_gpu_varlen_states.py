"""GPU parity of packed input with per-sequence initial and final states
(ssd_prefill_varlen_states through the C ABI; "Mamba-2炸裂升级！…", section "与vLLM的深度融合":
variable-length sequences and initial states without padding, one pseudo-chunk per sequence in
a chunk, handled by masking).  The oracle (oracle.recurrence_varlen_states) runs the fp64
recurrence over each sequence from its own initial state.  Layouts put sequences across many
chunks, starts on and between chunk starts, several starts in one chunk, one-token sequences,
and leave some sequence numbers unused (their final-state entries must stay untouched).
"""
import numpy as np
import pytest
import torch

import mamba_ssd_prefill_amd as ssd
import oracle
from gpu_common import DT_NAME, f64, fused_form, require_gpu, say
from mamba_ssd_prefill_amd.inputs import make_inputs
from parity import gate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def dev():
    return require_gpu()


def numbering(rows, L, order_seed=0):
    """int32 [B, L] from per-row lists of run lengths (the last run takes the rest); sequence
    numbers are a shuffled range so they do not follow token order, with number 1 left unused."""
    runs = []
    for lens in rows:
        used = sum(lens)
        assert used < L
        runs.append(list(lens) + [L - used])
    n = sum(len(r) for r in runs)
    rng = np.random.default_rng(order_seed)
    ids = [i for i in rng.permutation(n + 1) if i != 1][:n] if n >= 1 else []
    out = np.zeros((len(rows), L), dtype=np.int32)
    k = 0
    for b, r in enumerate(runs):
        t = 0
        for ln in r:
            out[b, t:t + ln] = ids[k]
            t += ln
            k += 1
    return torch.from_numpy(out), n + 1


def run(inp, seq, nseq, Q, impl, state_dtype, with_h0, seed):
    g = inp.to("cuda:0")
    H, P, N = inp.x.shape[2], inp.x.shape[3], inp.B.shape[3]
    h0 = None
    if with_h0:
        gen = torch.Generator().manual_seed(seed)
        h0 = (0.1 * torch.randn(nseq, H, P, N, generator=gen)).to(state_dtype)
    fin = torch.full((nseq, H, P, N), 7.0, dtype=state_dtype, device="cuda:0")  # sentinel
    with fused_form(impl) as name:
        y, fin = ssd.ssd_prefill_varlen_states(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, seq_idx=seq.to("cuda:0"),
                                               nseq=nseq, initial_states=None if h0 is None else h0.to("cuda:0"),
                                               chunk_size=Q, impl=name, state_dtype=state_dtype, final_states=fin)
    torch.cuda.synchronize()
    return y, fin, h0


def check(inp, seq, nseq, y, fin, h0, name):
    args = {k: v for k, v in inp.args().items() if k != "h0"}
    yr, fr = oracle.recurrence_varlen_states(**args, seq_idx=seq, nseq=nseq, initial_states=h0)
    in_dt = DT_NAME[inp.x.dtype]
    skip = f64(inp.D)[None, None, :, None] * f64(inp.x)
    gate(f64(y), yr, in_dt, in_dt, skip=skip, name=name + " y")
    used = ~np.isnan(fr[:, 0, 0, 0])
    gate(f64(fin)[used], fr[used], DT_NAME[fin.dtype], in_dt, name=name + " final states")
    assert bool((fin[torch.from_numpy(~used)] == 7.0).all()), name + ": an unused final-state entry was written"


def layouts(Q, L):
    # row 0: a start at token 1, one-token sequences, a run over several chunks, starts on a chunk
    # start and mid-chunk, three starts in one chunk, a start at the last token; row 1: two runs
    r0 = [1, Q - 1, 2 * Q + 5, 1, 1, 1, Q // 3, 17, Q - 9, 3]
    assert sum(r0) < L - 1
    r0 += [L - 1 - sum(r0)]  # then a run of length 1 at token L - 1
    return [r0, [Q + 19]]


@pytest.mark.parametrize("with_h0", [True, False])
@pytest.mark.parametrize("impl", ["unfused", "fused"])
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_varlen_states_bf16(Q, impl, with_h0):
    L = 6 * Q + 21
    inp = make_inputs(2, L, 8, 64, 128, 2, dtype="bf16", state_dtype="f32", has_h0=False, seed=9000 + Q)
    seq, nseq = numbering(layouts(Q, L), L, order_seed=Q)
    say("varlen states bf16 Q", Q, impl, with_h0)
    y, fin, h0 = run(inp, seq, nseq, Q, impl, torch.float32, with_h0, seed=Q)
    check(inp, seq, nseq, y, fin, h0, "varlen states bf16 Q%d %s h0=%s" % (Q, impl, with_h0))


@pytest.mark.parametrize("impl", ["unfused", "fused"])
def test_varlen_states_f16_with_f16_state(impl):
    Q, L = 128, 1000
    inp = make_inputs(1, L, 16, 64, 128, 1, dtype="f16", state_dtype="f16", has_h0=False, seed=9101)
    seq, nseq = numbering([[200, 1, 70, 128, 5, 300]], L, order_seed=3)
    say("varlen states f16/f16", impl)
    y, fin, h0 = run(inp, seq, nseq, Q, impl, torch.float16, True, seed=5)
    check(inp, seq, nseq, y, fin, h0, "varlen states f16/f16 %s" % impl)


@pytest.mark.parametrize("impl", ["unfused", "fused"])
@pytest.mark.parametrize("shape", [(32, 64, 4), (128, 128, 1), (16, 32, 2)], ids=["P32N64", "P128N128", "P16N32"])
def test_varlen_states_shapes_and_many_short(impl, shape):
    P, N, G = shape
    Q, L = 128, 900
    rng = np.random.default_rng(P + N)
    lens = [int(n) for n in rng.integers(1, 60, size=25)]
    lens = lens[:next(i for i in range(len(lens) + 1) if sum(lens[:i + 1]) >= L - 1 or i == len(lens))]
    inp = make_inputs(1, L, 8, P, N, G, dtype="bf16", state_dtype="f32", has_h0=False, seed=9200 + P)
    seq, nseq = numbering([lens], L, order_seed=P)
    say("varlen states shape", shape, impl, len(lens) + 1, "sequences")
    y, fin, h0 = run(inp, seq, nseq, Q, impl, torch.float32, True, seed=P)
    check(inp, seq, nseq, y, fin, h0, "varlen states %s %s" % (shape, impl))


def test_varlen_states_one_sequence_per_row_matches_prefill():
    """Each row one sequence, numbered by row: per-sequence states are then the per-row initial
    and final states of the plain prefill."""
    Q, L = 128, 700
    inp = make_inputs(3, L, 8, 64, 128, 2, dtype="bf16", state_dtype="f32", has_h0=True, seed=9300)
    seq = torch.arange(3, dtype=torch.int32)[:, None].repeat(1, L).contiguous()
    g = inp.to("cuda:0")
    y0, f0 = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q)
    y1, f1 = ssd.ssd_prefill_varlen_states(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, seq_idx=seq.to("cuda:0"), nseq=3,
                                           initial_states=g.h0, chunk_size=Q)
    torch.cuda.synchronize()
    gate(f64(y1), f64(y0), "bf16", "bf16", skip=f64(inp.D)[None, None, :, None] * f64(inp.x), name="rows y")
    gate(f64(f1), f64(f0), "f32", "bf16", name="rows final")
