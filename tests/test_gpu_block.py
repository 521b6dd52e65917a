"""GPU parity of the block form: the convolution before and the gated norm after the SSD
("Mamba-2炸裂升级！…", section "未来展望与应用拓展"), through the C ABI, against the oracle's
conv_silu / gated_rmsnorm / block (fp64).  The standalone kernels, the unfused block (three
kernels with the SSD's five between) and the fused block (convolution inside the launch) with
y sent to the norm kernel (the default) and with the norm inside the launch as well
(MAMBA_SSD_BLOCK_NORM=1, at shapes whose (b, g) pairs fall on whole work partitions).
"""
import os

import numpy as np
import pytest
import torch

import mamba_ssd_prefill_amd as ssd
import oracle
from gpu_common import DT_NAME, f64, require_gpu, say
from mamba_ssd_prefill_amd.inputs import make_block_inputs, make_inputs
from parity import gate

pytestmark = pytest.mark.gpu
EPS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def dev():
    return require_gpu()


def inputs(Bt, L, H, P, N, G, dtype="bf16", h0=True, state=True, seed=0):
    inp = make_inputs(Bt, L, H, P, N, G, dtype=dtype, state_dtype="f32", has_h0=h0, seed=seed)
    blk = make_block_inputs(Bt, L, H, P, N, G, dtype=dtype, has_state=state, seed=seed + 1)
    return inp, blk


def ref_block(inp, blk, H, P, G, N, dtype):
    return oracle.block(blk.xbc, blk.conv_w, blk.conv_b, blk.conv_state, inp.dt, inp.A, inp.D, inp.dt_bias, blk.z,
                        blk.norm_w, EPS, nheads=H, headdim=P, ngroups=G, dstate=N, h0=inp.h0, in_dtype=dtype)


def run_block(inp, blk, H, P, G, N, Q, impl):
    g, b = inp.to("cuda:0"), blk.to("cuda:0")
    out, fin = ssd.ssd_prefill_block(b.xbc, b.conv_w, b.conv_b, b.conv_state, g.dt, g.A, g.D, g.dt_bias, b.z,
                                     b.norm_w, EPS, g.h0, nheads=H, headdim=P, ngroups=G, dstate=N, chunk_size=Q,
                                     impl=impl)
    torch.cuda.synchronize()
    return out, fin


def test_conv_silu_kernel():
    Bt, L, H, P, N, G = 2, 77, 4, 64, 64, 2
    _, blk = inputs(Bt, L, H, P, N, G)
    b = blk.to("cuda:0")
    say("conv_silu %s" % ((Bt, L, H, P, N, G),))
    x, Bm, Cm = ssd.conv_silu(b.xbc, b.conv_w, b.conv_b, b.conv_state, nheads=H, headdim=P, ngroups=G, dstate=N)
    torch.cuda.synchronize()
    ref = oracle.conv_silu(blk.xbc, blk.conv_w, blk.conv_b, blk.conv_state)
    got = np.concatenate([f64(x).reshape(Bt, L, -1), f64(Bm).reshape(Bt, L, -1), f64(Cm).reshape(Bt, L, -1)], axis=2)
    # fp32 evaluation rounded once to bf16: within one bf16 rounding of the exact value
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


# (H, P, G): a group's pieces of 8 channels per lane of its wave are 1 (ragged), 2 (ragged), 4,
# 8, 10 (the 2.7B block's one group of 5120 channels) and 16 (the two-pass kernel)
@pytest.mark.parametrize("H,P,G", [(8, 64, 2), (25, 32, 1), (32, 64, 1), (64, 64, 1), (80, 64, 1),
                                   (128, 64, 1)], ids=lambda v: str(v))
def test_gated_norm_kernel(H, P, G):
    Bt, L = 2, 33
    gen = torch.Generator().manual_seed(5 + H + G)
    y = torch.randn(Bt, L, H * P, generator=gen).to(torch.bfloat16)
    z = torch.randn(Bt, L, H * P, generator=gen).to(torch.bfloat16)
    w = 1.0 + 0.1 * torch.randn(H * P, generator=gen)
    say("gated_norm H=%d P=%d G=%d" % (H, P, G))
    out = ssd.gated_norm(y.cuda(), z.cuda(), w.cuda(), EPS, nheads=H, headdim=P, ngroups=G)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(y, z, w, EPS, G)
    gate(f64(out), ref, "bf16", "bf16", name="gated_norm")


CASES = [
    # (B, L, H, P, N, G): the first two put whole (b, g) pairs on every partition (norm fused);
    # the others straddle partitions (norm kernel after the launch)
    (8, 300, 8, 64, 128, 1),
    (4, 200, 8, 64, 64, 2),
    (8, 150, 4, 128, 128, 1),
    (2, 333, 8, 64, 128, 2),
    (1, 520, 6, 64, 64, 1),
]


@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_block_fused(case, Q):
    Bt, L, H, P, N, G = case
    inp, blk = inputs(Bt, L, H, P, N, G, seed=hash(case) % 1000 + Q)
    say("block fused %s Q=%d" % (case, Q))
    out, fin = run_block(inp, blk, H, P, G, N, Q, "fused")
    rout, ry, rfin = ref_block(inp, blk, H, P, G, N, "bf16")
    gate(f64(out), rout, "bf16", "bf16", name="block out")
    gate(f64(fin), rfin, "f32", "bf16", name="block final")


@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: "_".join(map(str, c)))
def test_block_fused_norm_in_launch_and_unfused(case, Q, monkeypatch):
    Bt, L, H, P, N, G = case
    inp, blk = inputs(Bt, L, H, P, N, G, seed=11 + Q)
    rout, ry, rfin = ref_block(inp, blk, H, P, G, N, "bf16")
    say("block fused, norm in the launch %s Q=%d" % (case, Q))
    monkeypatch.setenv("MAMBA_SSD_BLOCK_NORM", "1")
    out, fin = run_block(inp, blk, H, P, G, N, Q, "fused")
    gate(f64(out), rout, "bf16", "bf16", name="block out (norm in the launch)")
    gate(f64(fin), rfin, "f32", "bf16", name="block final (norm in the launch)")
    monkeypatch.delenv("MAMBA_SSD_BLOCK_NORM")
    if Q != 128:
        return
    say("block unfused %s" % (case,))
    out, fin = run_block(inp, blk, H, P, G, N, 128, "unfused")
    gate(f64(out), rout, "bf16", "bf16", name="block out (unfused)")
    gate(f64(fin), rfin, "f32", "bf16", name="block final (unfused)")


def test_block_no_state_no_h0_f16():
    Bt, L, H, P, N, G = 8, 129, 8, 64, 128, 1
    inp, blk = inputs(Bt, L, H, P, N, G, dtype="f16", h0=False, state=False, seed=21)
    say("block f16 without states")
    out, fin = run_block(inp, blk, H, P, G, N, 128, "fused")
    rout, ry, rfin = ref_block(inp, blk, H, P, G, N, "f16")
    gate(f64(out), rout, "f16", "f16", name="block out f16")
    gate(f64(fin), rfin, "f32", "f16", name="block final f16")


def test_block_split_carries_both_states():
    """Two calls chained by the conv state (the first call's last 3 raw inputs) and the SSM state
    give the same out as one call."""
    Bt, L, H, P, N, G = 8, 256, 8, 64, 128, 1
    s = 100
    inp, blk = inputs(Bt, L, H, P, N, G, seed=31)
    say("block split")
    g, b = inp.to("cuda:0"), blk.to("cuda:0")
    kw = dict(nheads=H, headdim=P, ngroups=G, dstate=N, chunk_size=128, impl="fused")
    whole, fw = ssd.ssd_prefill_block(b.xbc, b.conv_w, b.conv_b, b.conv_state, g.dt, g.A, g.D, g.dt_bias, b.z,
                                      b.norm_w, EPS, g.h0, **kw)
    o1, f1 = ssd.ssd_prefill_block(b.xbc[:, :s].contiguous(), b.conv_w, b.conv_b, b.conv_state,
                                   g.dt[:, :s].contiguous(), g.A, g.D, g.dt_bias, b.z[:, :s].contiguous(), b.norm_w,
                                   EPS, g.h0, **kw)
    st = b.xbc[:, s - 3:s].permute(0, 2, 1).contiguous()
    o2, f2 = ssd.ssd_prefill_block(b.xbc[:, s:].contiguous(), b.conv_w, b.conv_b, st, g.dt[:, s:].contiguous(), g.A,
                                   g.D, g.dt_bias, b.z[:, s:].contiguous(), b.norm_w, EPS, f1, **kw)
    torch.cuda.synchronize()
    rout, ry, rfin = ref_block(inp, blk, H, P, G, N, "bf16")
    gate(f64(torch.cat([o1, o2], dim=1)), rout, "bf16", "bf16", name="split out")
    gate(f64(f2), rfin, "f32", "bf16", name="split final")
    gate(f64(whole), rout, "bf16", "bf16", name="whole out")


def test_block_refuses_unsupported():
    Bt, L, H, P, N, G = 1, 64, 4, 32, 64, 1
    inp, blk = inputs(Bt, L, H, P, N, G, seed=41)
    with pytest.raises(ssd.SSDError) as e:
        run_block(inp, blk, H, P, G, N, 128, "fused")
    assert e.value.code == 3  # SSD_ERR_UNSUPPORTED: headdim 32 has no fused block kernel
    out, fin = run_block(inp, blk, H, P, G, N, 128, "unfused")  # the unfused block takes it
    rout, ry, rfin = ref_block(inp, blk, H, P, G, N, "bf16")
    gate(f64(out), rout, "bf16", "bf16", name="unfused block P=32")


def test_block_norm_runs_inside_the_launch_where_pairs_are_whole():
    """The y region of the workspace (its last region) is left alone when the norm runs inside the
    launch (the chunk tiles write y to out, the norm items scale it there), and written when y
    goes to the norm kernel."""
    Bt, L, H, P, N, G = CASES[0]
    inp, blk = inputs(Bt, L, H, P, N, G, seed=51)
    g, b = inp.to("cuda:0"), blk.to("cuda:0")
    prm = ssd.make_params(Bt, L, H, P, N, G, 128, "bf16", "f32", True, "fused")
    total = ssd.block_workspace_size(prm)
    ysz = (Bt * L * H * P * 2 + 255) // 256 * 256
    touched = {}
    for norm in ("1", "0"):
        os.environ["MAMBA_SSD_BLOCK_NORM"] = norm
        try:
            ws = torch.full((total,), 0xFF, dtype=torch.uint8, device="cuda:0")
            say("block y region, MAMBA_SSD_BLOCK_NORM=%s" % norm)
            ssd.ssd_prefill_block(b.xbc, b.conv_w, b.conv_b, b.conv_state, g.dt, g.A, g.D, g.dt_bias, b.z, b.norm_w,
                                  EPS, g.h0, nheads=H, headdim=P, ngroups=G, dstate=N, chunk_size=128, impl="fused",
                                  workspace=ws)
            torch.cuda.synchronize()
            touched[norm] = bool((ws[total - ysz:] != 0xFF).any())
        finally:
            del os.environ["MAMBA_SSD_BLOCK_NORM"]
    assert touched == {"1": False, "0": True}  # 1: norm items in the launch; 0 (default): norm kernel


@pytest.mark.parametrize("norm", ["0", "1"])
def test_block_2p7b_full_every_row(norm, monkeypatch):
    """The fused block at the 2.7B layer shape (B=8, L=8192, H=80, P=64, N=128, G=1, Q=128; every
    batch row is one work partition, so the norm can run inside the launch), with the norm kernel
    and with the norm in the launch, compared with the oracle's block row by row on every element
    of out and of the final state."""
    monkeypatch.setenv("MAMBA_SSD_BLOCK_NORM", norm)
    from mamba_ssd_prefill_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["mamba2_2p7b_bf16"]
    Bt, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    inp = workload_inputs(w)
    blk = make_block_inputs(Bt, L, H, P, N, G, dtype=w.dtype, has_state=True, seed=2003)
    say("block 2.7B full size")
    out, fin = run_block(inp, blk, H, P, G, N, 128, "fused")
    out, fin = f64(out), f64(fin)
    for b in range(Bt):
        row = lambda t: None if t is None else t[b:b + 1].contiguous()  # noqa: E731
        rout, ry, rfin = oracle.block(row(blk.xbc), blk.conv_w, blk.conv_b, row(blk.conv_state), row(inp.dt), inp.A,
                                      inp.D, inp.dt_bias, row(blk.z), blk.norm_w, EPS, nheads=H, headdim=P, ngroups=G,
                                      dstate=N, h0=row(inp.h0), in_dtype=w.dtype)
        gate(out[b:b + 1], rout, "bf16", "bf16", name="2.7B block out row %d" % b)
        gate(fin[b:b + 1], rfin, "f32", "bf16", name="2.7B block final row %d" % b)
