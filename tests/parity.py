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
    rep = {"name": name, "max_abs_err": float(err.max()) if err.size else 0.0,
           "core_scale": scale,
           "normalised_err": float((err / max(scale, 1e-30)).max()) if err.size else 0.0}
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise ParityError("%s: contract tolerance exceeded at %s: got %r ref %r (%d elements)"
                          % (name, i, got[i], ref[i], int(bad.sum())))
    if bad2.any():
        i = np.unravel_index(np.argmax(err - lim2), err.shape)
        raise ParityError("%s: normalised check failed at %s: got %r ref %r err %.3g > %.3g (%d elements)"
                          % (name, i, got[i], ref[i], err[i], lim2[i], int(bad2.sum())))
    return rep
