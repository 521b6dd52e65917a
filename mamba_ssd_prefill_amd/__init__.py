"""MI355X-native Mamba-2 SSD chunked prefill (forward).

A thin ctypes binding over libmamba_ssd.so (C ABI in include/mamba_ssd.h).  Every step
of the computation runs in the library's HIP kernels; this module only marshals
arguments.  PyTorch provides device memory and the stream.  If the library is not
built, every call raises: there is no fallback path.

    y, final_state = ssd_prefill(x, dt, A, B, C, D, dt_bias, initial_state,
                                 chunk_size=128, impl="fused")
"""
import ctypes
import os

__all__ = ["ssd_prefill", "workspace_size", "workspace_layout", "Params", "SSDError", "library_path",
           "load_library", "step_chunk_cumsum", "step_bmm", "step_chunk_state", "step_state_passing",
           "step_chunk_scan", "check_device_status", "make_params", "ssd_decode_step", "ssd_prefill_noalloc",
           "ssd_prefill_varlen_states", "conv_silu", "gated_norm", "ssd_prefill_block", "block_workspace_size",
           "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("MAMBA_SSD_LIB", os.path.join(_HERE, "libmamba_ssd.so"))

SSD_F32, SSD_F16, SSD_BF16 = 0, 1, 2
DTYPE_CODES = {"f32": SSD_F32, "f16": SSD_F16, "bf16": SSD_BF16}
IMPL_CODES = {"unfused": 0, "fused": 1}
FLAG_WORKSPACE_READY = 1  # ssd_params_t.flags bit: see ssd_prefill(workspace_ready=...)
STATUS_NAMES = {0: "SSD_OK", 1: "SSD_ERR_NULL_POINTER", 2: "SSD_ERR_INVALID_SHAPE", 3: "SSD_ERR_UNSUPPORTED",
                4: "SSD_ERR_MISALIGNED", 5: "SSD_ERR_WORKSPACE_TOO_SMALL", 6: "SSD_ERR_HIP",
                7: "SSD_ERR_SYNC_TIMEOUT", 8: "SSD_ERR_INVALID_ARGUMENT", 9: "SSD_ERR_SCHEDULE",
                10: "SSD_ERR_SCRATCH_TOO_SMALL"}
EXPORTED_SYMBOLS = ["ssd_prefill_workspace_size", "ssd_validate", "ssd_prefill", "ssd_prefill_timed",
                    "ssd_check_device_status",
                    "ssd_status_string", "ssd_workspace_layout", "ssd_step_chunk_cumsum", "ssd_step_bmm",
                    "ssd_step_chunk_state", "ssd_step_state_passing", "ssd_step_chunk_scan", "ssd_decode_step",
                    "ssd_prefill_varlen", "ssd_prefill_noalloc", "ssd_prefill_varlen_states", "ssd_conv_silu",
                    "ssd_gated_norm", "ssd_prefill_block_workspace_size", "ssd_prefill_block"]


class SSDError(RuntimeError):
    def __init__(self, code, where=""):
        self.code = code
        msg = STATUS_NAMES.get(code, str(code))
        try:
            msg += ": " + load_library().ssd_status_string(code).decode()
        except Exception:  # pragma: no cover
            pass
        super().__init__("%s%s" % (where + ": " if where else "", msg))


class Params(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_size_t), ("batch", ctypes.c_int), ("seqlen", ctypes.c_int),
                ("nheads", ctypes.c_int), ("headdim", ctypes.c_int), ("dstate", ctypes.c_int),
                ("ngroups", ctypes.c_int), ("chunk_size", ctypes.c_int), ("in_dtype", ctypes.c_int),
                ("state_dtype", ctypes.c_int), ("dt_softplus", ctypes.c_int), ("impl", ctypes.c_int),
                ("relaxed", ctypes.c_int), ("flags", ctypes.c_int)]


class Layout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("dt_offset", ctypes.c_size_t), ("acs_offset", ctypes.c_size_t),
                ("cb_offset", ctypes.c_size_t), ("s_offset", ctypes.c_size_t), ("states_offset", ctypes.c_size_t),
                ("sync_offset", ctypes.c_size_t), ("status_offset", ctypes.c_size_t), ("dt_bytes", ctypes.c_size_t),
                ("acs_bytes", ctypes.c_size_t), ("cb_bytes", ctypes.c_size_t), ("s_bytes", ctypes.c_size_t),
                ("states_bytes", ctypes.c_size_t), ("sync_bytes", ctypes.c_size_t), ("nchunks", ctypes.c_int),
                ("state_slots", ctypes.c_int), ("seg_offset", ctypes.c_size_t), ("seg_bytes", ctypes.c_size_t)]


_lib = None


def library_path():
    return _LIB_PATH


def load_library():
    """Load libmamba_ssd.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libmamba_ssd.so is not built (%s); run `python -m mamba_ssd_prefill_amd.build`"
                           % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Params)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.ssd_prefill_workspace_size.argtypes = [P]
    lib.ssd_prefill_workspace_size.restype = sz
    lib.ssd_validate.argtypes = [P]
    lib.ssd_validate.restype = ctypes.c_int
    lib.ssd_prefill.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_prefill.restype = ctypes.c_int
    lib.ssd_prefill_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.ssd_prefill_varlen.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_prefill_varlen.restype = ctypes.c_int
    lib.ssd_prefill_timed.restype = ctypes.c_int
    lib.ssd_check_device_status.argtypes = [P, vp, vp]
    lib.ssd_check_device_status.restype = ctypes.c_int
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_workspace_layout.argtypes = [P, ctypes.POINTER(Layout)]
    lib.ssd_workspace_layout.restype = ctypes.c_int
    lib.ssd_step_chunk_cumsum.argtypes = [P, vp, vp, vp, vp, sz, vp]
    lib.ssd_step_bmm.argtypes = [P, vp, vp, vp, sz, vp]
    lib.ssd_step_chunk_state.argtypes = [P, vp, vp, vp, sz, vp]
    lib.ssd_step_state_passing.argtypes = [P, vp, vp, vp, sz, vp]
    lib.ssd_step_chunk_scan.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.ssd_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_prefill_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_prefill_noalloc.restype = ctypes.c_int
    lib.ssd_prefill_varlen_states.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, sz, vp]
    lib.ssd_prefill_varlen_states.restype = ctypes.c_int
    fl = ctypes.c_float
    lib.ssd_conv_silu.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_gated_norm.argtypes = [P, vp, vp, vp, fl, vp, vp]
    lib.ssd_prefill_block_workspace_size.argtypes = [P]
    lib.ssd_prefill_block_workspace_size.restype = sz
    lib.ssd_prefill_block.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, fl, vp, vp, vp, vp, sz, vp]
    for f in ("ssd_step_chunk_cumsum", "ssd_step_bmm", "ssd_step_chunk_state", "ssd_step_state_passing",
              "ssd_step_chunk_scan", "ssd_decode_step", "ssd_conv_silu", "ssd_gated_norm", "ssd_prefill_block"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _dtype_code(t):
    import torch
    return {torch.float32: SSD_F32, torch.float16: SSD_F16, torch.bfloat16: SSD_BF16}[t.dtype]


def make_params(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size=128, in_dtype="bf16",
                state_dtype="f32", dt_softplus=True, impl="fused", relaxed=False, flags=0):
    code = lambda d: d if isinstance(d, int) else DTYPE_CODES[d]  # noqa: E731
    return Params(ctypes.sizeof(Params), int(batch), int(seqlen), int(nheads), int(headdim), int(dstate),
                  int(ngroups), int(chunk_size), code(in_dtype), code(state_dtype), 1 if dt_softplus else 0,
                  IMPL_CODES[impl] if isinstance(impl, str) else int(impl), 1 if relaxed else 0, int(flags))


def _params_for(x, B, chunk_size, state_dtype_code, dt_softplus, impl, relaxed=False, flags=0):
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return make_params(Bt, L, H, P, N, G, chunk_size, _dtype_code(x), state_dtype_code, dt_softplus, impl, relaxed,
                       flags)


def workspace_size(params):
    n = load_library().ssd_prefill_workspace_size(ctypes.byref(params))
    if n == 0:
        raise SSDError(load_library().ssd_validate(ctypes.byref(params)), "ssd_prefill_workspace_size")
    return n


def workspace_layout(params):
    out = Layout()
    rc = load_library().ssd_workspace_layout(ctypes.byref(params), ctypes.byref(out))
    if rc:
        raise SSDError(rc, "ssd_workspace_layout")
    return out


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(rc, where):
    if rc != 0:
        raise SSDError(rc, where)


def alloc_workspace(params, device):
    import torch
    return torch.empty(workspace_size(params), dtype=torch.uint8, device=device)


def _check_tensors(x, dt, A, B, C, D, dt_bias, h0):
    import torch
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_prefill needs device tensors (got %s)" % dev)
    want = {"dt": (dt, (Bt, L, H)), "B": (B, (Bt, L, G, N)), "C": (C, (Bt, L, G, N)), "A": (A, (H,)),
            "D": (D, (H,)), "dt_bias": (dt_bias, (H,)), "initial_state": (h0, (Bt, H, P, N))}
    for name, (t, shape) in want.items():
        if t is None:
            continue
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if t.device != dev:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    for name, t in (("dt", dt), ("B", B), ("C", C)):
        if t.dtype != x.dtype:
            raise ValueError("%s must have x's dtype %s" % (name, x.dtype))
    for name, t in (("A", A), ("D", D), ("dt_bias", dt_bias)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError("%s must be float32" % name)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")


def ssd_prefill(x, dt, A, B, C, D=None, dt_bias=None, initial_state=None, chunk_size=128, state_dtype=None,
                impl="fused", dt_softplus=True, workspace=None, y=None, final_state=None, kernel_events=None,
                seq_idx=None, relaxed=False, workspace_ready=False):
    """Run one SSD prefill on the GPU; returns (y[B,L,H,P], final_state[B,H,P,N]).

    ``state_dtype`` defaults to initial_state's dtype, else float32.  ``workspace``
    (uint8 device tensor), ``y`` and ``final_state`` may be passed to avoid allocation.
    ``kernel_events`` = (begin, end) torch.cuda.Event(enable_timing=True) pair, recorded
    by the library around the SSD compute kernel(s) (ssd_prefill_timed).  ``seq_idx``
    (int32 [B, L]) packs several sequences per batch row: the recurrence restarts wherever
    it changes (ssd_prefill_varlen).  ``relaxed``: CB stored in the 16-bit input type.
    ``workspace_ready``: SSD_FLAG_WORKSPACE_READY -- ``workspace`` is untouched since the previous
    call with the same arguments' shapes and types (the library then skips the launch that
    resets it when there is no initial state; it checks that the previous call matches)."""
    import torch
    _check_tensors(x, dt, A, B, C, D, dt_bias, initial_state)
    if seq_idx is not None:
        if (tuple(seq_idx.shape) != tuple(x.shape[:2]) or seq_idx.dtype != torch.int32 or seq_idx.device != x.device
                or not seq_idx.is_contiguous()):
            raise ValueError("seq_idx must be a contiguous int32 [B, L] tensor on %s" % x.device)
        if kernel_events is not None:
            raise ValueError("kernel_events are not recorded for packed variable-length input")
    if state_dtype is None:
        state_dtype = initial_state.dtype if initial_state is not None else torch.float32
    sd = {torch.float32: SSD_F32, torch.float16: SSD_F16, torch.bfloat16: SSD_BF16}[state_dtype]
    if initial_state is not None and initial_state.dtype != state_dtype:
        raise ValueError("initial_state dtype %s != state_dtype %s" % (initial_state.dtype, state_dtype))
    if workspace_ready and workspace is None:
        raise ValueError("workspace_ready needs the workspace of the previous call")
    prm = _params_for(x, B, chunk_size, sd, dt_softplus, impl, relaxed, FLAG_WORKSPACE_READY if workspace_ready else 0)
    Bt, L, H, P = x.shape
    N = B.shape[3]
    if y is None:
        y = torch.empty_like(x)
    if final_state is None:
        final_state = torch.empty((Bt, H, P, N), dtype=state_dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(prm, x.device)
    args = (ctypes.byref(prm), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
            _ptr(initial_state), _ptr(y), _ptr(final_state), _ptr(workspace), workspace.numel(), _stream(x.device))
    if seq_idx is not None:
        _check(load_library().ssd_prefill_varlen(*args[:8], _ptr(seq_idx), *args[8:]), "ssd_prefill_varlen")
    elif kernel_events is None:
        _check(load_library().ssd_prefill(*args), "ssd_prefill")
    else:
        ev0, ev1 = kernel_events
        for ev in (ev0, ev1):
            if ev.cuda_event == 0:  # torch creates the HIP event lazily on first record
                ev.record()
        _check(load_library().ssd_prefill_timed(*args, ctypes.c_void_p(ev0.cuda_event), ctypes.c_void_p(ev1.cuda_event)),
               "ssd_prefill_timed")
    return y, final_state


def ssd_prefill_varlen_states(x, dt, A, B, C, D=None, dt_bias=None, seq_idx=None, nseq=None, initial_states=None,
                              chunk_size=128, state_dtype=None, impl="fused", dt_softplus=True, workspace=None,
                              y=None, final_states=None, relaxed=False):
    """Packed sequences with a state per sequence (ssd_prefill_varlen_states): seq_idx (int32
    [B, L]) numbers the sequence of each token, in [0, nseq); ``initial_states`` (None: zeros)
    and the returned ``final_states`` are [nseq, H, P, N].  Returns (y, final_states)."""
    import torch
    _check_tensors(x, dt, A, B, C, D, dt_bias, None)
    if seq_idx is None or nseq is None:
        raise ValueError("seq_idx and nseq are required")
    if (tuple(seq_idx.shape) != tuple(x.shape[:2]) or seq_idx.dtype != torch.int32 or seq_idx.device != x.device
            or not seq_idx.is_contiguous()):
        raise ValueError("seq_idx must be a contiguous int32 [B, L] tensor on %s" % x.device)
    Bt, L, H, P = x.shape
    N = B.shape[3]
    if state_dtype is None:
        state_dtype = initial_states.dtype if initial_states is not None else torch.float32
    for name, t in (("initial_states", initial_states), ("final_states", final_states)):
        if t is not None and (tuple(t.shape) != (nseq, H, P, N) or t.dtype != state_dtype or t.device != x.device
                              or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous %s [%d, %d, %d, %d] tensor" % (name, state_dtype, nseq, H, P, N))
    sd = {torch.float32: SSD_F32, torch.float16: SSD_F16, torch.bfloat16: SSD_BF16}[state_dtype]
    prm = _params_for(x, B, chunk_size, sd, dt_softplus, impl, relaxed)
    if y is None:
        y = torch.empty_like(x)
    if final_states is None:
        final_states = torch.zeros((nseq, H, P, N), dtype=state_dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(prm, x.device)
    _check(load_library().ssd_prefill_varlen_states(
        ctypes.byref(prm), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(seq_idx),
        int(nseq), _ptr(initial_states), _ptr(y), _ptr(final_states), _ptr(workspace), workspace.numel(),
        _stream(x.device)), "ssd_prefill_varlen_states")
    return y, final_states


def ssd_prefill_noalloc(x, dt, A, B, C, D=None, dt_bias=None, initial_state=None, chunk_size=128, state_dtype=None,
                        impl="fused", dt_softplus=True, y=None, final_state=None):
    """ssd_prefill through ssd_prefill_noalloc: the library's static scratch is the workspace, so
    the call allocates no device memory when ``y`` and ``final_state`` are passed (this binding
    allocates them with torch only when they are not).  Returns (y, final_state)."""
    import torch
    _check_tensors(x, dt, A, B, C, D, dt_bias, initial_state)
    if state_dtype is None:
        state_dtype = initial_state.dtype if initial_state is not None else torch.float32
    sd = {torch.float32: SSD_F32, torch.float16: SSD_F16, torch.bfloat16: SSD_BF16}[state_dtype]
    prm = _params_for(x, B, chunk_size, sd, dt_softplus, impl)
    Bt, L, H, P = x.shape
    N = B.shape[3]
    if y is None:
        y = torch.empty_like(x)
    if final_state is None:
        final_state = torch.empty((Bt, H, P, N), dtype=state_dtype, device=x.device)
    _check(load_library().ssd_prefill_noalloc(ctypes.byref(prm), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                              _ptr(dt_bias), _ptr(initial_state), _ptr(y), _ptr(final_state),
                                              _stream(x.device)), "ssd_prefill_noalloc")
    return y, final_state


def _block_params(xbc, dt, nheads, headdim, ngroups, dstate, chunk_size, state_dtype, dt_softplus, impl):
    import torch
    Bt, L, ch = xbc.shape
    if ch != nheads * headdim + 2 * ngroups * dstate:
        raise ValueError("xbc has %d channels, expected H*P + 2*G*N = %d" % (ch, nheads * headdim + 2 * ngroups * dstate))
    if tuple(dt.shape) != (Bt, L, nheads):
        raise ValueError("dt must be [B, L, H]")
    sd = {torch.float32: SSD_F32, torch.float16: SSD_F16, torch.bfloat16: SSD_BF16}[state_dtype]
    return make_params(Bt, L, nheads, headdim, dstate, ngroups, chunk_size, _dtype_code(xbc), sd, dt_softplus, impl)


def _device_contig(*ts):
    for t in ts:
        if t is not None and (t.device.type != "cuda" or not t.is_contiguous()):
            raise ValueError("the block entry points need contiguous device tensors")


def conv_silu(xbc, conv_w, conv_b=None, conv_state=None, *, nheads, headdim, ngroups, dstate):
    """ssd_conv_silu: x [B, L, H, P], B and C [B, L, G, N] from xbc [B, L, H*P + 2*G*N]."""
    import torch
    _device_contig(xbc, conv_w, conv_b, conv_state)
    Bt, L, _ = xbc.shape
    prm = make_params(Bt, L, nheads, headdim, dstate, ngroups, 128, _dtype_code(xbc), SSD_F32, True, "unfused")
    x = torch.empty((Bt, L, nheads, headdim), dtype=xbc.dtype, device=xbc.device)
    Bm = torch.empty((Bt, L, ngroups, dstate), dtype=xbc.dtype, device=xbc.device)
    Cm = torch.empty_like(Bm)
    _check(load_library().ssd_conv_silu(ctypes.byref(prm), _ptr(xbc), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state),
                                        _ptr(x), _ptr(Bm), _ptr(Cm), _stream(xbc.device)), "ssd_conv_silu")
    return x, Bm, Cm


def gated_norm(y, z, norm_w, norm_eps, *, nheads, headdim, ngroups, out=None):
    """ssd_gated_norm: out [B, L, H*P] = the gated RMS norm of y (y, z [B, L, H, P] or [B, L, H*P])."""
    import torch
    _device_contig(y, z, norm_w, out)
    Bt, L = y.shape[:2]
    hp = nheads * headdim
    prm = make_params(Bt, L, nheads, headdim, 32, ngroups, 128, _dtype_code(y), SSD_F32, True, "unfused")
    if out is None:
        out = torch.empty((Bt, L, hp), dtype=y.dtype, device=y.device)
    _check(load_library().ssd_gated_norm(ctypes.byref(prm), _ptr(y), _ptr(z), _ptr(norm_w), float(norm_eps), _ptr(out),
                                         _stream(y.device)), "ssd_gated_norm")
    return out


def block_workspace_size(params):
    n = load_library().ssd_prefill_block_workspace_size(ctypes.byref(params))
    if n == 0:
        raise SSDError(3, "ssd_prefill_block_workspace_size")
    return n


def ssd_prefill_block(xbc, conv_w, conv_b, conv_state, dt, A, D, dt_bias, z, norm_w, norm_eps, initial_state=None, *,
                      nheads, headdim, ngroups, dstate, chunk_size=128, state_dtype=None, impl="fused",
                      dt_softplus=True, workspace=None, out=None, final_state=None):
    """ssd_prefill_block: the convolution, the SSD prefill and the gated norm.  Returns
    (out [B, L, H*P], final_state [B, H, P, N])."""
    import torch
    _device_contig(xbc, conv_w, conv_b, conv_state, dt, A, D, dt_bias, z, norm_w, initial_state, out, final_state)
    if state_dtype is None:
        state_dtype = initial_state.dtype if initial_state is not None else torch.float32
    prm = _block_params(xbc, dt, nheads, headdim, ngroups, dstate, chunk_size, state_dtype, dt_softplus, impl)
    Bt, L, _ = xbc.shape
    if out is None:
        out = torch.empty((Bt, L, nheads * headdim), dtype=xbc.dtype, device=xbc.device)
    if final_state is None:
        final_state = torch.empty((Bt, nheads, headdim, dstate), dtype=state_dtype, device=xbc.device)
    if workspace is None:
        workspace = torch.empty(block_workspace_size(prm), dtype=torch.uint8, device=xbc.device)
    _check(load_library().ssd_prefill_block(
        ctypes.byref(prm), _ptr(xbc), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(dt), _ptr(A), _ptr(D),
        _ptr(dt_bias), _ptr(z), _ptr(norm_w), float(norm_eps), _ptr(initial_state), _ptr(out), _ptr(final_state),
        _ptr(workspace), workspace.numel(), _stream(xbc.device)), "ssd_prefill_block")
    return out, final_state


def check_device_status(params, workspace):
    rc = load_library().ssd_check_device_status(ctypes.byref(params), _ptr(workspace), _stream(workspace.device))
    return rc


# ---- per-step entry points (unfused form) ------------------------------------------------------
def step_chunk_cumsum(params, dt, A, dt_bias, workspace):
    _check(load_library().ssd_step_chunk_cumsum(ctypes.byref(params), _ptr(dt), _ptr(A), _ptr(dt_bias),
                                                _ptr(workspace), workspace.numel(), _stream(dt.device)),
           "ssd_step_chunk_cumsum")


def step_bmm(params, B, C, workspace):
    _check(load_library().ssd_step_bmm(ctypes.byref(params), _ptr(B), _ptr(C), _ptr(workspace), workspace.numel(),
                                       _stream(B.device)), "ssd_step_bmm")


def step_chunk_state(params, x, B, workspace):
    _check(load_library().ssd_step_chunk_state(ctypes.byref(params), _ptr(x), _ptr(B), _ptr(workspace),
                                               workspace.numel(), _stream(x.device)), "ssd_step_chunk_state")


def step_state_passing(params, initial_state, final_state, workspace):
    _check(load_library().ssd_step_state_passing(ctypes.byref(params), _ptr(initial_state), _ptr(final_state),
                                                 _ptr(workspace), workspace.numel(), _stream(workspace.device)),
           "ssd_step_state_passing")


def step_chunk_scan(params, x, C, D, y, workspace):
    _check(load_library().ssd_step_chunk_scan(ctypes.byref(params), _ptr(x), _ptr(C), _ptr(D), _ptr(y),
                                              _ptr(workspace), workspace.numel(), _stream(x.device)),
           "ssd_step_chunk_scan")


# ---- single-token decode step ----------------------------------------------------------------
def ssd_decode_step(x, dt, A, B, C, D=None, dt_bias=None, state=None, state_dtype=None, dt_softplus=True,
                    out_state=None, y=None):
    """One token of the recurrence per batch row on a cached state (ssd_decode_step in the C
    ABI); returns (y[B,H,P], new_state[B,H,P,N]).

    x [B,H,P], dt [B,H], B and C [B,G,N] (x's dtype); A, D, dt_bias [H] float32; ``state``
    [B,H,P,N] (None: zeros) in ``state_dtype`` (default: state's dtype, else float32).
    ``out_state`` receives the new state (default: ``state`` itself, updated in place, or a
    new tensor when ``state`` is None)."""
    import torch
    Bt, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_decode_step needs device tensors (got %s)" % dev)
    if state_dtype is None:
        state_dtype = state.dtype if state is not None else torch.float32
    want = {"dt": (dt, (Bt, H)), "B": (B, (Bt, G, N)), "C": (C, (Bt, G, N)), "A": (A, (H,)), "D": (D, (H,)),
            "dt_bias": (dt_bias, (H,)), "state": (state, (Bt, H, P, N)), "out_state": (out_state, (Bt, H, P, N)),
            "y": (y, (Bt, H, P))}
    for name, (t, shape) in want.items():
        if t is None:
            continue
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if t.device != dev or not t.is_contiguous():
            raise ValueError("%s must be a contiguous tensor on %s" % (name, dev))
    for name, t in (("dt", dt), ("B", B), ("C", C), ("y", y)):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("%s must have x's dtype %s" % (name, x.dtype))
    for name, t in (("state", state), ("out_state", out_state)):
        if t is not None and t.dtype != state_dtype:
            raise ValueError("%s dtype %s != state_dtype %s" % (name, t.dtype, state_dtype))
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    sd = {torch.float32: SSD_F32, torch.float16: SSD_F16, torch.bfloat16: SSD_BF16}[state_dtype]
    prm = make_params(Bt, 1, H, P, N, G, 128, _dtype_code(x), sd, dt_softplus, "fused")
    if out_state is None:
        out_state = state if state is not None else torch.empty((Bt, H, P, N), dtype=state_dtype, device=dev)
    if y is None:
        y = torch.empty_like(x)
    _check(load_library().ssd_decode_step(ctypes.byref(prm), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                          _ptr(dt_bias), _ptr(state), _ptr(out_state), _ptr(y), _stream(dev)),
           "ssd_decode_step")
    return y, out_state
