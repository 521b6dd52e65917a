"""GPU parity of packed variable-length prefill (ssd_prefill_varlen through the C ABI).

Several sequences share a batch row, told apart by a per-token sequence index and masked
("Mamba-2炸裂升级！…", section "与vLLM的深度融合").  The oracle runs the fp64 recurrence over
each sequence on its own (oracle.recurrence_varlen); every comparison goes through the
parity gate.  Layouts put sequence starts on chunk starts, in the middle of chunks, several
in one chunk, at the last token, and include sequences of length 1.
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


def seq_index(lengths_per_row, L):
    """int32 [B, L]: row b holds sequences of the given lengths (the last one takes the rest)."""
    out = np.zeros((len(lengths_per_row), L), dtype=np.int32)
    for b, lens in enumerate(lengths_per_row):
        t, sid = 0, 0
        for n in lens:
            out[b, t:t + n] = sid
            t += n
            sid += 1
        out[b, t:] = sid
        assert t <= L
    return torch.from_numpy(out)


def layouts(Q, L):
    # row 0: starts at chunk starts, mid-chunk, several per chunk, length-1 sequences, a start at
    # the last token; row 1: one sequence (no start inside the row)
    r0 = [1, Q - 1, Q, 3, 1, 2, 2 * Q + 5, 17, Q // 2]
    used = sum(r0)
    assert used < L - 1
    r0 += [L - 1 - used]  # then one more sequence of length 1 at token L - 1
    return [r0, []]


def run_varlen(inp, seq, Q, impl, state_dtype=None):
    with fused_form(impl) as name:
        g = inp.to("cuda:0")
        sd = state_dtype or (g.h0.dtype if g.h0 is not None else torch.float32)
        Bt, L, H, P = g.x.shape
        G, N = g.B.shape[2], g.B.shape[3]
        prm = ssd.make_params(Bt, L, H, P, N, G, Q, DT_NAME[g.x.dtype], DT_NAME[sd], inp.dt_softplus, name)
        ws = ssd.alloc_workspace(prm, g.x.device)
        y, fin = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q, impl=name,
                                 state_dtype=sd, workspace=ws, seq_idx=seq.to("cuda:0"))
        torch.cuda.synchronize()
        assert ssd.check_device_status(prm, ws) == 0
        return y, fin


def check(inp, seq, y, fin, name):
    yr, fr = oracle.recurrence_varlen(**inp.args(), seq_idx=seq)
    in_dt = DT_NAME[inp.x.dtype]
    skip = f64(inp.D)[None, None, :, None] * f64(inp.x) if inp.D is not None else None
    gate(f64(y), yr, in_dt, in_dt, skip=skip, name=name + " y")
    gate(f64(fin), fr, DT_NAME[fin.dtype], in_dt, name=name + " final")


IMPLS = ["unfused", "fused_hop", "fused_relay2", "fused_relay4"]


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("Q", [64, 128, 256])
def test_varlen_bf16(Q, impl):
    L = 5 * Q + 37
    inp = make_inputs(2, L, 8, 64, 128, 2, dtype="bf16", state_dtype="f32", has_h0=True, seed=8000 + Q)
    seq = seq_index(layouts(Q, L), L)
    say("varlen bf16 Q", Q, impl)
    y, fin = run_varlen(inp, seq, Q, impl)
    check(inp, seq, y, fin, "varlen bf16 Q%d %s" % (Q, impl))


@pytest.mark.parametrize("impl", ["unfused", "fused_hop", "fused_relay2"])
def test_varlen_f16_with_f16_state(impl):
    Q, L = 128, 700
    inp = make_inputs(1, L, 16, 64, 128, 1, dtype="f16", state_dtype="f16", has_h0=True, seed=8101)
    seq = seq_index([[200, 1, 70, 128, 5]], L)
    say("varlen f16 state", impl)
    y, fin = run_varlen(inp, seq, Q, impl)
    check(inp, seq, y, fin, "varlen f16/f16 %s" % impl)


@pytest.mark.parametrize("impl", ["unfused", "fused_hop", "fused_relay2"])
def test_varlen_f32(impl):
    Q, L = 64, 300
    inp = make_inputs(2, L, 4, 16, 16, 1, dtype="f32", state_dtype="f32", has_h0=True, seed=8102)
    seq = seq_index([[64, 90, 1, 40], [150]], L)
    say("varlen f32", impl)
    y, fin = run_varlen(inp, seq, Q, impl)
    check(inp, seq, y, fin, "varlen f32 %s" % impl)


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("shape", [(16, 16), (32, 64)], ids=["P16N16", "P32N64"])
def test_varlen_f32_dozens_of_starts_per_chunk(impl, shape):
    """fp32 inputs held to the fp32 contract (1e-5) with up to 31 sequence starts in one chunk:
    30 sequences of one token, then longer ones, so later sequences of a chunk sit behind many
    starts (the masked decays must lose nothing to them)."""
    P, N = shape
    Q, L = 64, 400
    lens = [1] * 30 + [34, 2, 3, 1, 1, 5, 60, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 9, 100]
    inp = make_inputs(2, L, 4, P, N, 1, dtype="f32", state_dtype="f32", has_h0=True, seed=8105 + P)
    seq = seq_index([lens, [3] * 20 + [250]], L)
    say("varlen f32 many starts", shape, impl)
    y, fin = run_varlen(inp, seq, Q, impl)
    check(inp, seq, y, fin, "varlen f32 many starts %s %s" % (shape, impl))


@pytest.mark.parametrize("impl", ["unfused", "fused_hop", "fused_relay2"])
def test_varlen_grouped_many_short_sequences(impl):
    # grouped B/C (4 heads per group), 24 sequences of 1..80 tokens in one row, no initial state
    Q, L = 128, 1000
    rng = np.random.default_rng(5)
    lens = []
    for n in rng.integers(1, 81, size=64):
        if sum(lens) + int(n) >= L - 1 or len(lens) == 23:
            break
        lens.append(int(n))
    inp = make_inputs(1, L, 16, 64, 128, 4, dtype="bf16", state_dtype="f32", has_h0=False, seed=8103)
    seq = seq_index([lens], L)
    say("varlen grouped", impl)
    y, fin = run_varlen(inp, seq, Q, impl)
    check(inp, seq, y, fin, "varlen grouped %s" % impl)


@pytest.mark.parametrize("impl", ["unfused", "fused"])
def test_one_sequence_per_row_is_bitwise_the_plain_prefill(impl):
    Q, L = 128, 600
    inp = make_inputs(2, L, 8, 64, 128, 2, dtype="bf16", state_dtype="f32", has_h0=True, seed=8104)
    seq = torch.full((2, L), 7, dtype=torch.int32)
    y1, f1 = run_varlen(inp, seq, Q, impl)
    g = inp.to("cuda:0")
    with fused_form(impl) as name:
        y2, f2 = ssd.ssd_prefill(g.x, g.dt, g.A, g.B, g.C, g.D, g.dt_bias, g.h0, chunk_size=Q, impl=name)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("impl", ["fused", "unfused"])
def test_packed_short_sequences_full_size(impl):
    """The bench's packed workload at full size: the 32 x 1024-token short-sequence batch (H=128,
    G=8, bf16, Q=128) packed into one row of 32768 tokens with seq_idx.  Sampled heads, every
    token, against the oracle run on each sampled head alone (a head reads only its own x, dt,
    A, D, dt_bias and its group's B and C)."""
    from mamba_ssd_prefill_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["short_g8_bf16"]
    inp = workload_inputs(w)
    Bt, L, H = w.batch, w.seqlen, w.nheads
    hpg = H // w.ngroups
    packed = make_inputs(1, 1, H, w.headdim, w.dstate, w.ngroups, dtype=w.dtype, seed=0)
    packed.x, packed.dt = inp.x.reshape(1, Bt * L, H, -1), inp.dt.reshape(1, Bt * L, H)
    packed.B, packed.C = inp.B.reshape(1, Bt * L, w.ngroups, -1), inp.C.reshape(1, Bt * L, w.ngroups, -1)
    packed.A, packed.D, packed.dt_bias, packed.h0 = inp.A, inp.D, inp.dt_bias, None
    seq = torch.arange(Bt, dtype=torch.int32).repeat_interleave(L).reshape(1, Bt * L).contiguous()
    say("packed short sequences", impl)
    y, fin = run_varlen(packed, seq, w.chunk_size, impl)
    for h in (0, 17, 64, 127):
        g = h // hpg
        one = make_inputs(1, 1, 1, w.headdim, w.dstate, 1, dtype=w.dtype, seed=0)
        one.x, one.dt = packed.x[:, :, h:h + 1].contiguous(), packed.dt[:, :, h:h + 1].contiguous()
        one.B, one.C = packed.B[:, :, g:g + 1].contiguous(), packed.C[:, :, g:g + 1].contiguous()
        one.A, one.D, one.dt_bias, one.h0 = packed.A[h:h + 1], packed.D[h:h + 1], packed.dt_bias[h:h + 1], None
        yr, fr = oracle.recurrence_varlen(**one.args(), seq_idx=seq)
        skip = f64(one.D)[None, None, :, None] * f64(one.x)
        gate(f64(y[:, :, h:h + 1]), yr, "bf16", "bf16", skip=skip, name="packed %s head %d y" % (impl, h))
        gate(f64(fin[:, h:h + 1]), fr, "f32", "bf16", name="packed %s head %d final" % (impl, h))
