"""fp64 CPU oracle for the Mamba-2 SSD chunked prefill.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library never
imports, links or calls it, and it shares no code with the HIP library.

* ``recurrence``  -- the definition: the sequential per-token recurrence (C, fp64).
* ``chunked``     -- the five-step chunked algorithm with its intermediates (C, fp64).
* ``quadratic``   -- the brute-force masked-matrix form (numpy, fp64, tiny inputs).
* ``decode_step`` -- one token of the recurrence on a cached state (the decode step).
* ``recurrence_varlen`` -- packed variable-length input: the recurrence restarted at every
  sequence start.
* ``recurrence_varlen_states`` -- packed input with per-sequence initial and final states.
* ``conv_silu``, ``gated_rmsnorm``, ``block`` -- the convolution before and the norm after
  the SSD, and the three composed.

Inputs may be torch CPU tensors or numpy arrays; 16-bit tensors are passed to C
as their raw bits and widened exactly there.
"""
import ctypes
import os
import subprocess

import numpy as np

from .quadratic import ssd_quadratic  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")

_DT_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def build(force=False):
    """Compile the C oracle with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int), ("seqlen", ctypes.c_int), ("nheads", ctypes.c_int),
        ("headdim", ctypes.c_int), ("dstate", ctypes.c_int), ("ngroups", ctypes.c_int),
        ("in_dtype", ctypes.c_int), ("state_dtype", ctypes.c_int), ("dt_softplus", ctypes.c_int),
        ("x", ctypes.c_void_p), ("dt", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("Bm", ctypes.c_void_p), ("Cm", ctypes.c_void_p), ("D", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p), ("h0", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        dp = ctypes.POINTER(ctypes.c_double)
        lib.ssd_oracle_recurrence.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(ctypes.c_int),
                                              ctypes.c_int, dp, dp, ctypes.c_int, dp]
        lib.ssd_oracle_recurrence.restype = ctypes.c_int
        lib.ssd_oracle_chunked.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, dp, dp, dp, dp, dp, dp, dp]
        lib.ssd_oracle_chunked.restype = ctypes.c_int
        lib.ssd_oracle_widen.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_long, dp]
        lib.ssd_oracle_widen.restype = None
        lib.ssd_oracle_num_threads.argtypes = []
        lib.ssd_oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads():
    return _load().ssd_oracle_num_threads()


def _dtype_name(a):
    """Element dtype name of a torch tensor or numpy array."""
    s = str(a.dtype)
    if "bfloat16" in s:
        return "bf16"
    if "float16" in s:
        return "f16"
    if "float32" in s:
        return "f32"
    raise TypeError("unsupported dtype %s" % s)


def _raw(a, keep):
    """Contiguous host buffer holding the element bits of ``a``; returns its address."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            t = a.detach().cpu().contiguous()
            if t.dtype in (torch.bfloat16, torch.float16):
                arr = t.view(torch.int16).numpy()
            else:
                arr = t.numpy()
            keep.append(arr)
            return arr.ctypes.data
    except ImportError:  # pragma: no cover
        pass
    arr = np.ascontiguousarray(a)
    keep.append(arr)
    return arr.ctypes.data


def _f32(a, keep):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            arr = a.detach().cpu().to(torch.float32).contiguous().numpy()
            keep.append(arr)
            return arr.ctypes.data
    except ImportError:  # pragma: no cover
        pass
    arr = np.ascontiguousarray(a, dtype=np.float32)
    keep.append(arr)
    return arr.ctypes.data


def _problem(x, dt, A, B, C, D, dt_bias, h0, dt_softplus, keep):
    Bt, L, H, P = (int(s) for s in x.shape)
    G, N = int(B.shape[2]), int(B.shape[3])
    in_dt = _dtype_name(x)
    for t in (dt, B, C):
        if _dtype_name(t) != in_dt:
            raise TypeError("x, dt, B and C must share one dtype")
    st_dt = _dtype_name(h0) if h0 is not None else "f32"
    pr = _Problem(Bt, L, H, P, N, G, _DT_CODE[in_dt], _DT_CODE[st_dt], 1 if dt_softplus else 0,
                  _raw(x, keep), _raw(dt, keep), _f32(A, keep), _raw(B, keep), _raw(C, keep),
                  _f32(D, keep), _f32(dt_bias, keep), _raw(h0, keep))
    return pr, (Bt, L, H, P, N, G)


def _dptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrence(x, dt, A, B, C, D=None, dt_bias=None, h0=None, dt_softplus=True,
               bh=None, snap_q=0, want_y=True):
    """Sequential fp64 recurrence for the (b, h) pairs in ``bh`` (default: all).

    Returns ``(y[nbh, L, P], final[nbh, P, N], snaps)``; ``snaps`` is
    ``[nbh, ceil(L/snap_q), P, N]`` (state after each snap_q tokens) or None."""
    keep = []
    pr, (Bt, L, H, P, N, G) = _problem(x, dt, A, B, C, D, dt_bias, h0, dt_softplus, keep)
    if bh is None:
        bh = [(b, h) for b in range(Bt) for h in range(H)]
    flat = np.ascontiguousarray([b * H + h for (b, h) in bh], dtype=np.int32)
    nbh = len(flat)
    y = np.empty((nbh, L, P)) if want_y else None
    fin = np.empty((nbh, P, N))
    snaps = np.empty((nbh, (L + snap_q - 1) // snap_q, P, N)) if snap_q > 0 else None
    rc = _load().ssd_oracle_recurrence(ctypes.byref(pr), flat.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                                       nbh, _dptr(y), _dptr(fin), int(snap_q), _dptr(snaps))
    if rc != 0:
        raise ValueError("ssd_oracle_recurrence rejected its arguments")
    return y, fin, snaps


def recurrence_full(x, dt, A, B, C, D=None, dt_bias=None, h0=None, dt_softplus=True):
    """All (b, h) pairs, reshaped to y[B, L, H, P] and final[B, H, P, N]."""
    Bt, L, H, P = (int(s) for s in x.shape)
    N = int(B.shape[3])
    y, fin, _ = recurrence(x, dt, A, B, C, D, dt_bias, h0, dt_softplus)
    return y.reshape(Bt, H, L, P).transpose(0, 2, 1, 3).copy(), fin.reshape(Bt, H, P, N)


def chunked(x, dt, A, B, C, D=None, dt_bias=None, h0=None, dt_softplus=True, chunk_size=64):
    """Five-step chunked fp64 evaluation; returns a dict of every intermediate."""
    keep = []
    pr, (Bt, L, H, P, N, G) = _problem(x, dt, A, B, C, D, dt_bias, h0, dt_softplus, keep)
    Q = int(chunk_size)
    nc = (L + Q - 1) // Q
    out = {
        "dt": np.empty((Bt, nc, H, Q)),
        "acs": np.empty((Bt, nc, H, Q)),
        "cb": np.empty((Bt, nc, G, Q, Q)),
        "s": np.empty((Bt, nc, H, P, N)),
        "states": np.empty((Bt, nc + 1, H, P, N)),
        "y": np.empty((Bt, L, H, P)),
        "final": np.empty((Bt, H, P, N)),
    }
    rc = _load().ssd_oracle_chunked(ctypes.byref(pr), Q, _dptr(out["dt"]), _dptr(out["acs"]), _dptr(out["cb"]),
                                    _dptr(out["s"]), _dptr(out["states"]), _dptr(out["y"]), _dptr(out["final"]))
    if rc != 0:
        raise ValueError("ssd_oracle_chunked rejected its arguments")
    return out


def decode_step(x, dt, A, B, C, D=None, dt_bias=None, state=None, dt_softplus=True):
    """One autoregressive step: the recurrence over a single token per batch row, started from
    ``state`` ("Mamba-2状态空间模型的编译器优化与实现", section 2.1: the cached [B,H,P,N] state is
    updated once per generated token).  x [B,H,P], dt [B,H], B/C [B,G,N], state [B,H,P,N] or
    None (zeros).  Returns ``(y[B,H,P], new_state[B,H,P,N])`` in fp64."""
    Bt, H, P = (int(s) for s in x.shape)
    G, N = int(B.shape[1]), int(B.shape[2])
    y, fin = recurrence_full(x.reshape(Bt, 1, H, P), dt.reshape(Bt, 1, H), A, B.reshape(Bt, 1, G, N),
                             C.reshape(Bt, 1, G, N), D, dt_bias, state, dt_softplus)
    return y.reshape(Bt, H, P), fin


def recurrence_varlen(x, dt, A, B, C, D=None, dt_bias=None, h0=None, dt_softplus=True, seq_idx=None):
    """Several sequences packed in each batch row ("Mamba-2炸裂升级！…", section "与vLLM的深度融合"):
    a new sequence starts at every t > 0 where seq_idx[b, t] != seq_idx[b, t-1], and the
    recurrence runs over each sequence on its own -- the first sequence of row b from h0[b],
    every later one from zero.  Returns y[B, L, H, P] and the state after the last token of
    each row, [B, H, P, N], in fp64."""
    Bt, L, H, P = (int(s) for s in x.shape)
    N = int(B.shape[3])
    sidx = np.asarray(seq_idx.cpu() if hasattr(seq_idx, "cpu") else seq_idx)
    y = np.empty((Bt, L, H, P))
    fin = np.empty((Bt, H, P, N))
    for b in range(Bt):
        starts = [0] + [t for t in range(1, L) if sidx[b, t] != sidx[b, t - 1]] + [L]
        for k in range(len(starts) - 1):
            t0, t1 = starts[k], starts[k + 1]
            part = lambda t: None if t is None else t[b:b + 1, t0:t1].contiguous()  # noqa: E731
            init = h0[b:b + 1] if (h0 is not None and k == 0) else None
            yk, fk = recurrence_full(part(x), part(dt), A, part(B), part(C), D, dt_bias, init, dt_softplus)
            y[b, t0:t1] = yk[0]
            fin[b] = fk[0]
    return y, fin


def widen(t):
    """Exact fp64 values of a 16-bit or fp32 tensor, decoded by the oracle's own C code."""
    keep = []
    code = _DT_CODE[_dtype_name(t)]
    ptr = _raw(t, keep)
    n = int(np.prod(t.shape))
    out = np.empty(n)
    _load().ssd_oracle_widen(ctypes.c_void_p(ptr), code, n, _dptr(out))
    return out.reshape(tuple(t.shape))


def recurrence_varlen_states(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True, seq_idx=None, nseq=0,
                             initial_states=None):
    """Packed sequences with a state per sequence ("Mamba-2炸裂升级！…", section "与vLLM的深度融合":
    variable-length sequences and initial states without padding).  A sequence starts at t = 0
    of every row and wherever seq_idx changes; seq_idx[b, t] in [0, nseq) is its number.
    Sequence q runs the recurrence from initial_states[q] (or zero) over its tokens;
    final_states[q] is its state after its last token.  Returns y[B, L, H, P] and
    final_states[nseq, H, P, N] in fp64 (NaN for numbers no run uses)."""
    Bt, L, H, P = (int(s) for s in x.shape)
    N = int(B.shape[3])
    sidx = np.asarray(seq_idx.cpu() if hasattr(seq_idx, "cpu") else seq_idx)
    y = np.empty((Bt, L, H, P))
    fin = np.full((int(nseq), H, P, N), np.nan)
    for b in range(Bt):
        starts = [0] + [t for t in range(1, L) if sidx[b, t] != sidx[b, t - 1]] + [L]
        for k in range(len(starts) - 1):
            t0, t1 = starts[k], starts[k + 1]
            q = int(sidx[b, t0])
            part = lambda t: None if t is None else t[b:b + 1, t0:t1].contiguous()  # noqa: E731
            init = initial_states[q:q + 1] if initial_states is not None else None
            yk, fk = recurrence_full(part(x), part(dt), A, part(B), part(C), D, dt_bias, init, dt_softplus)
            y[b, t0:t1] = yk[0]
            fin[q] = fk[0]
    return y, fin


def _f64(a):
    """Exact fp64 values of a torch tensor / numpy array (16-bit types decoded by ``widen``)."""
    if a is None:
        return None
    if hasattr(a, "cpu"):  # torch tensor
        import torch
        if a.dtype in (torch.float16, torch.bfloat16):
            return widen(a)
        return a.detach().cpu().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def conv_silu(xbc, conv_w, conv_b=None, conv_state=None):
    """The causal depthwise convolution before the SSD, then SiLU ("Mamba-2炸裂升级！…", section
    "Mamba-2核心操作与融合的必要性": the depthwise convolution mixes the last few tokens; section
    "未来展望与应用拓展": the convolution before the SSD).  Per channel ch and token t, with K the
    width (conv_w [Ch, K]):

        v[b,t,ch]   = conv_b[ch] + sum_k conv_w[ch,k] * in[b, t-(K-1)+k, ch]
        out[b,t,ch] = v / (1 + exp(-v))

    where in[b, t<0, ch] = conv_state[b, ch, t+K-1] (the K-1 inputs before token 0, the decode
    cache's conv state of "Mamba-2状态空间模型的编译器优化与实现", section 2.2), zeros when
    conv_state is None.  xbc [B, L, Ch]; returns fp64 [B, L, Ch]."""
    x = _f64(xbc)
    w = _f64(conv_w)
    Bt, L, Ch = x.shape
    K = w.shape[1]
    prev = np.zeros((Bt, K - 1, Ch)) if conv_state is None else np.transpose(_f64(conv_state), (0, 2, 1))
    full = np.concatenate([prev, x], axis=1)  # token t of the input is row t + K - 1
    v = np.zeros((Bt, L, Ch)) if conv_b is None else np.broadcast_to(_f64(conv_b), (Bt, L, Ch)).copy()
    for k in range(K):
        v += w[:, k] * full[:, k:k + L, :]
    return v / (1.0 + np.exp(-v))


def gated_rmsnorm(y, z, norm_w, eps, ngroups):
    """The norm after the SSD ("Mamba-2炸裂升级！…", section "未来展望与应用拓展"), read as Mamba-2's
    gated RMS norm: g = y * silu(z) over the H*P channels of a token, normalised over each of
    ngroups contiguous channel groups, scaled per channel:

        out[b,t,c] = g[b,t,c] / sqrt(mean_{c' in group(c)} g[b,t,c']^2 + eps) * norm_w[c]

    y, z [B, L, H*P] (or [B, L, H, P]); returns fp64 [B, L, H*P]."""
    yv = _f64(y)
    Bt, L = yv.shape[:2]
    yv = yv.reshape(Bt, L, -1)
    zv = _f64(z).reshape(Bt, L, -1)
    C = yv.shape[2]
    g = yv * (zv / (1.0 + np.exp(-zv)))
    gg = g.reshape(Bt, L, ngroups, C // ngroups)
    ms = np.mean(gg * gg, axis=3, keepdims=True)
    return (gg / np.sqrt(ms + eps)).reshape(Bt, L, C) * _f64(norm_w)


def block(xbc, conv_w, conv_b, conv_state, dt, A, D, dt_bias, z, norm_w, eps, nheads, headdim, ngroups, dstate,
          h0=None, dt_softplus=True, in_dtype=None):
    """The SSD with the convolution before it and the norm after it (the fusion the same section
    describes): conv_silu over xBC = [x | B | C] (channels h*P + p, then H*P + g*N + n, then
    H*P + G*N + g*N + n), the conv output rounded to the input dtype (the SSD's operands are in
    that dtype), the recurrence, then gated_rmsnorm with one norm group per B/C group.
    Returns (out [B, L, H*P], y [B, L, H, P], final [B, H, P, N]) in fp64."""
    import torch
    H, P, G, N = nheads, headdim, ngroups, dstate
    xc = conv_silu(xbc, conv_w, conv_b, conv_state)
    Bt, L, _ = xc.shape
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[in_dtype or _dtype_name(xbc)]
    xr = torch.from_numpy(xc).to(torch.float32).to(tdt)  # rounded as a kernel writing fp32 results would
    HP = H * P
    x = xr[..., :HP].reshape(Bt, L, H, P).contiguous()
    Bm = xr[..., HP:HP + G * N].reshape(Bt, L, G, N).contiguous()
    Cm = xr[..., HP + G * N:HP + 2 * G * N].reshape(Bt, L, G, N).contiguous()
    y, fin = recurrence_full(x, dt, A, Bm, Cm, D, dt_bias, h0, dt_softplus)
    out = gated_rmsnorm(y, z, norm_w, eps, G)
    return out, y, fin
