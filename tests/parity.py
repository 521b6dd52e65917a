"""The parity gate every GPU-vs-oracle comparison goes through.

Two checks, both on every element:

1. the contract tolerance: fp32 inputs max|gpu - ref| <= 1e-5; fp16/bf16 inputs
   |gpu - ref| <= 1e-2 + 1e-2 |ref|;
2. a normalised check that still bites when the D x skip term dominates |y|:
   |gpu - ref| <= u(ref) + tau * max|ref - D x| for y, and
   |gpu - ref| <= u(ref) + tau * max|ref| for the final state, where u(ref) is
   half an ulp of the stored dtype at |ref| (the rounding every stored value has)
   and tau = 1e-2 for 16-bit inputs, 1e-4 for fp32 inputs.

tests/test_gate_discriminates.py shows on the CPU that plausible kernel mistakes
fail this gate while a correct evaluation rounded to the output dtypes passes.

``StreamGate`` applies the same two checks to an array fed in blocks (torch float64 on
the host, multithreaded), so full-size outputs are compared element by element without
holding the whole fp64 reference at once; tests/test_parity_stream.py checks that it
takes the same decisions as ``gate``.
"""
import numpy as np

_MANT = {"f32": 23, "f16": 10, "bf16": 7}
_EMIN = {"f32": -126, "f16": -14, "bf16": -126}
CONTRACT = {"f32": (1e-5, 0.0), "f16": (1e-2, 1e-2), "bf16": (1e-2, 1e-2)}
TAU = {"f32": 1e-4, "f16": 1e-2, "bf16": 1e-2}


def half_ulp(ref, dtype):
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** _EMIN[dtype])))
    return np.ldexp(1.0, (e - _MANT[dtype] - 1).astype(np.int64))


class ParityError(AssertionError):
    pass


def gate(got, ref, dtype, in_dtype, skip=None, name="y"):
    """Raise ParityError unless ``got`` matches ``ref``; returns a small report.

    ``dtype`` is the stored dtype of ``got``; ``in_dtype`` selects the tolerances;
    ``skip`` is the D x term (for y) or None (for the final state)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ParityError("%s: shape %s != %s" % (name, got.shape, ref.shape))
    if not np.all(np.isfinite(got)):
        raise ParityError("%s: non-finite values" % name)
    err = np.abs(got - ref)
    atol, rtol = CONTRACT[in_dtype]
    bad = err > atol + rtol * np.abs(ref)
    core = ref - skip if skip is not None else ref
    scale = float(np.max(np.abs(core))) if core.size else 0.0
    lim2 = half_ulp(ref, dtype) + TAU[in_dtype] * scale
    bad2 = err > lim2
    hu = half_ulp(ref, dtype)
    rep = {"name": name, "max_abs_err": float(err.max()) if err.size else 0.0,
           "core_scale": scale,
           "normalised_err": float((err / max(scale, 1e-30)).max()) if err.size else 0.0,
           # the error left after the rounding of the stored output itself (the part the
           # kernel's arithmetic is responsible for)
           "normalised_err_net": float((np.maximum(err - hu, 0.0) / max(scale, 1e-30)).max()) if err.size else 0.0}
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise ParityError("%s: contract tolerance exceeded at %s: got %r ref %r (%d elements)"
                          % (name, i, got[i], ref[i], int(bad.sum())))
    if bad2.any():
        i = np.unravel_index(np.argmax(err - lim2), err.shape)
        raise ParityError("%s: normalised check failed at %s: got %r ref %r err %.3g > %.3g (%d elements)"
                          % (name, i, got[i], ref[i], err[i], lim2[i], int(bad2.sum())))
    return rep


class StreamGate:
    """``gate`` over an array delivered in blocks: ``add(got, ref, skip)`` per block (any
    shapes, torch tensors or numpy arrays), then ``finish()`` raises ParityError or returns
    the report.  The contract check is elementwise; the normalised check needs the scale of
    the whole array, so each block keeps its largest ``err - half_ulp(ref)`` and the
    comparison with ``tau * scale`` happens at the end."""

    def __init__(self, dtype, in_dtype, name="y"):
        self.dtype, self.in_dtype, self.name = dtype, in_dtype, name
        self.scale = 0.0
        self.max_err = 0.0
        self.worst2 = -np.inf   # largest err - half_ulp(ref)
        self.worst2_at = None
        self.n = 0
        self.block = 0

    @staticmethod
    def _t(a):
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu", torch.float64)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))

    def _half_ulp(self, ref):
        """half_ulp() from the fp64 exponent field: |ref| = 1.m 2^(E - 1023) for normal values,
        so floor(log2 |ref|) = E - 1023 (E clamped below at the dtype's smallest normal)."""
        import torch
        E = ref.abs().view(torch.int64) >> 52
        E = torch.clamp(E, min=_EMIN[self.dtype] + 1023)
        return ((E - (_MANT[self.dtype] + 1)) << 52).view(torch.float64)

    def add(self, got, ref, skip=None):
        import torch
        got, ref = self._t(got), self._t(ref)
        if got.shape != ref.shape:
            raise ParityError("%s: block shape %s != %s" % (self.name, tuple(got.shape), tuple(ref.shape)))
        if not bool(torch.isfinite(got).all()):
            raise ParityError("%s: non-finite values in block %d" % (self.name, self.block))
        err = (got - ref).abs()
        atol, rtol = CONTRACT[self.in_dtype]
        over = err - (atol + rtol * ref.abs())
        if bool((over > 0).any()):
            i = np.unravel_index(int(torch.argmax(over)), tuple(err.shape))
            raise ParityError("%s: contract tolerance exceeded in block %d at %s: got %r ref %r (%d elements)"
                              % (self.name, self.block, i, float(got[i]), float(ref[i]), int((over > 0).sum())))
        core = ref - self._t(skip) if skip is not None else ref
        if core.numel():
            self.scale = max(self.scale, float(core.abs().max()))
            self.max_err = max(self.max_err, float(err.max()))
            d = err - self._half_ulp(ref)
            k = int(torch.argmax(d))
            if float(d.reshape(-1)[k]) > self.worst2:
                self.worst2 = float(d.reshape(-1)[k])
                i = np.unravel_index(k, tuple(err.shape))
                self.worst2_at = (self.block, i, float(got[i]), float(ref[i]))
        self.n += err.numel()
        self.block += 1

    def finish(self):
        lim = TAU[self.in_dtype] * self.scale
        if self.n and self.worst2 > lim:
            raise ParityError("%s: normalised check failed at block %d %s: got %r ref %r err - half_ulp %.3g > %.3g"
                              % ((self.name,) + self.worst2_at + (self.worst2, lim)))
        sc = max(self.scale, 1e-30)
        return {"name": self.name, "elements": self.n, "max_abs_err": self.max_err, "core_scale": self.scale,
                "normalised_err_net": max(self.worst2, 0.0) / sc}
