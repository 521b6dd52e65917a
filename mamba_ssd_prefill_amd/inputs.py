"""Seeded synthetic inputs for the SSD prefill workloads.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, so both the HIP path's tests and the oracle may use it.

Workloads follow the sizes the kernel-fusion write-up benchmarks ("Mamba-2炸裂升级！…",
section "实测数据惊艳亮相": batch 1-32, sequence length 1K-256K, fp16 state) at the
layer shapes of Mamba-2 130M and 2.7B.  Value recipe (the same for every workload):

* x ~ N(0, 1); B, C ~ N(0, 1) / sqrt(N)
* dt_raw ~ N(0, 1); per head a target step dt* = exp(U[ln 1e-3, ln 1e-1]) and
  dt_bias = dt* + log(-expm1(-dt*)) (the inverse of softplus at dt*), so
  softplus(0 + dt_bias) = dt*: per-head steps log-uniform in [1e-3, 1e-1]
* A = -exp(U[0, ln 16]) in [-16, -1]; D ~ N(0, 1)
* h0 ~ 0.1 * N(0, 1) where the workload has an initial state, else None

Draw order, from ``torch.Generator().manual_seed(seed)``: x, B, C, dt_raw, dt*, A,
D, h0.  Values are drawn in fp32 and rounded to nearest-even into the input dtype.
"""
from dataclasses import dataclass, field, replace
import math
from typing import Optional

import torch

_TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    dtype: str           # x, dt, B, C, y
    state_dtype: str     # h0, final state, inter-chunk states
    has_h0: bool
    seed: int
    chunk_sweep: tuple = field(default=())

    @property
    def tokens(self):
        return self.batch * self.seqlen

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", 1, 256, 4, 16, 16, 1, 64, "f32", "f32", False, 1001),
        Workload("mamba2_130m_f16", 1, 4096, 24, 64, 128, 1, 128, "f16", "f32", False, 1002),
        Workload("mamba2_2p7b_bf16", 8, 8192, 80, 64, 128, 1, 128, "bf16", "f32", True, 1003,
                 chunk_sweep=(64, 128, 256)),
        Workload("long_131k_f16", 1, 131072, 80, 64, 128, 1, 128, "f16", "f16", True, 1004),
        Workload("long_262k_f16", 1, 262144, 80, 64, 128, 1, 128, "f16", "f16", True, 1004),
        Workload("short_g8_bf16", 32, 1024, 128, 64, 128, 8, 128, "bf16", "f32", False, 1005),
    ]
}


@dataclass
class SSDInputs:
    x: torch.Tensor                  # [B, L, H, P]
    dt: torch.Tensor                 # [B, L, H] (raw, before bias / softplus)
    A: torch.Tensor                  # [H] fp32
    B: torch.Tensor                  # [B, L, G, N]
    C: torch.Tensor                  # [B, L, G, N]
    D: Optional[torch.Tensor]        # [H] fp32
    dt_bias: Optional[torch.Tensor]  # [H] fp32
    h0: Optional[torch.Tensor]       # [B, H, P, N] state dtype
    dt_softplus: bool = True

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return SSDInputs(mv(self.x), mv(self.dt), mv(self.A), mv(self.B), mv(self.C),
                         mv(self.D), mv(self.dt_bias), mv(self.h0), self.dt_softplus)

    def args(self):
        return dict(x=self.x, dt=self.dt, A=self.A, B=self.B, C=self.C, D=self.D,
                    dt_bias=self.dt_bias, h0=self.h0, dt_softplus=self.dt_softplus)


def make_inputs(batch, seqlen, nheads, headdim, dstate, ngroups, dtype="bf16",
                state_dtype="f32", has_h0=False, seed=0, with_D=True):
    """Draw one problem following the module recipe (see the module docstring)."""
    g = torch.Generator().manual_seed(int(seed))
    tdt = _TORCH_DT[dtype]
    x = torch.randn(batch, seqlen, nheads, headdim, generator=g)
    scale = 1.0 / math.sqrt(dstate)
    Bm = torch.randn(batch, seqlen, ngroups, dstate, generator=g).mul_(scale)
    Cm = torch.randn(batch, seqlen, ngroups, dstate, generator=g).mul_(scale)
    dt_raw = torch.randn(batch, seqlen, nheads, generator=g)
    u = torch.rand(nheads, generator=g)
    dt_target = torch.exp(math.log(1e-3) + u * (math.log(1e-1) - math.log(1e-3)))
    dt_bias = dt_target + torch.log(-torch.expm1(-dt_target))
    A = -torch.exp(torch.rand(nheads, generator=g) * math.log(16.0))
    D = torch.randn(nheads, generator=g)
    h0 = None
    if has_h0:
        h0 = (0.1 * torch.randn(batch, nheads, headdim, dstate, generator=g)).to(_TORCH_DT[state_dtype])
    return SSDInputs(x.to(tdt), dt_raw.to(tdt), A.float(), Bm.to(tdt), Cm.to(tdt),
                     D.float() if with_D else None, dt_bias.float(), h0)


def workload_inputs(w: Workload, seed=None, **overrides):
    """Inputs for a named workload (sizes may be overridden, e.g. a shorter seqlen)."""
    w = w.with_(**overrides) if overrides else w
    return make_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                       w.dtype, w.state_dtype, w.has_h0, w.seed if seed is None else seed)


@dataclass
class BlockInputs:
    """The block form's extra inputs (the convolution before and the gated norm after the SSD);
    dt, A, D, dt_bias and h0 come from an SSDInputs of the same shape."""
    xbc: "object"         # [B, L, H*P + 2*G*N], input dtype
    conv_w: "object"      # [H*P + 2*G*N, 4] fp32
    conv_b: "object"      # [H*P + 2*G*N] fp32
    conv_state: "object"  # [B, H*P + 2*G*N, 3] input dtype, or None
    z: "object"           # [B, L, H*P] input dtype
    norm_w: "object"      # [H*P] fp32

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device).contiguous()  # noqa: E731
        return BlockInputs(mv(self.xbc), mv(self.conv_w), mv(self.conv_b), mv(self.conv_state), mv(self.z),
                           mv(self.norm_w))


def make_block_inputs(batch, seqlen, nheads, headdim, dstate, ngroups, dtype="bf16", has_state=True, seed=0):
    """Recipe: the raw x channels of xBC ~ N(0, 1), the raw B and C channels ~ N(0, 1) / sqrt(N)
    (the plain recipe's scale); taps ~ N(0, 0.5^2), bias ~ N(0, 0.1^2); the conv state drawn like
    xBC's channels; z ~ N(0, 1); norm weights 1 + 0.1 N(0, 1).  Draw order from
    ``torch.Generator().manual_seed(seed)``: xbc, conv_w, conv_b, conv_state, z, norm_w."""
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    gen = torch.Generator().manual_seed(seed)
    hp, gn = nheads * headdim, ngroups * dstate
    ch = hp + 2 * gn
    scale = torch.cat([torch.ones(hp), torch.full((2 * gn,), 1.0 / math.sqrt(dstate))])
    xbc = (torch.randn(batch, seqlen, ch, generator=gen) * scale).to(tdt)
    conv_w = 0.5 * torch.randn(ch, 4, generator=gen)
    conv_b = 0.1 * torch.randn(ch, generator=gen)
    st = (torch.randn(batch, 3, ch, generator=gen) * scale).permute(0, 2, 1).contiguous().to(tdt)
    z = torch.randn(batch, seqlen, hp, generator=gen).to(tdt)
    norm_w = 1.0 + 0.1 * torch.randn(hp, generator=gen)
    return BlockInputs(xbc, conv_w, conv_b, st if has_state else None, z, norm_w)
