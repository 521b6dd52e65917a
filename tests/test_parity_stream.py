"""StreamGate (blocks of a large array) must take the same decisions as gate() (whole array).

CPU only.  Cases: a correct rounded evaluation, an error spread thinly over one block, one
element over the contract tolerance, and the normalised check failing only because of the
scale the other blocks set.
"""
import numpy as np
import pytest
import torch

from parity import ParityError, StreamGate, gate, half_ulp


def _round(a, dtype):
    t = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(a).to(t).to(torch.float64).numpy()


def _decide(fn):
    try:
        fn()
        return True
    except ParityError:
        return False


def _both(got, ref, skip, dtype, in_dtype, nblocks):
    whole = _decide(lambda: gate(got, ref, dtype, in_dtype, skip=skip))

    def streamed():
        sg = StreamGate(dtype, in_dtype)
        for gb, rb, sb in zip(np.array_split(got, nblocks), np.array_split(ref, nblocks),
                              np.array_split(skip, nblocks) if skip is not None else [None] * nblocks):
            sg.add(gb, rb, sb)
        return sg.finish()

    return whole, _decide(streamed)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("nblocks", [1, 3, 7])
def test_stream_matches_gate(dtype, nblocks):
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((21, 40)) * 0.05
    skip = rng.standard_normal((21, 40)) * 3.0
    full = ref + skip
    good = _round(full, dtype)
    assert _both(good, full, skip, dtype, dtype, nblocks) == (True, True)

    # one block off by a small relative amount: fails the normalised check only
    bad = good.copy()
    bad[10:12] += 0.03 * np.max(np.abs(ref)) if dtype != "f32" else 3e-4 * np.max(np.abs(ref))
    w, s = _both(bad, full, skip, dtype, dtype, nblocks)
    assert w == s

    # one element above the contract tolerance
    bad = good.copy()
    bad[20, 39] += 0.5
    assert _both(bad, full, skip, dtype, dtype, nblocks) == (False, False)


def test_scale_comes_from_all_blocks():
    """An error that the scale of the whole array rejects must be rejected even when the block
    holding it has a large local scale and the other blocks a small one (and vice versa)."""
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((8, 50)) * 1e-3
    ref[0, 0] = 1.0                      # block 0 sets the scale
    got = ref.copy()
    got[7, 3] += 5e-3                    # below 1e-2 * 1.0: passes with the whole-array scale
    assert _both(got, ref, None, "f32", "bf16", 4) == (True, True)
    got[7, 3] += 2e-2                    # above it
    assert _both(got, ref, None, "f32", "bf16", 4) == (False, False)


def test_half_ulp_matches_numpy():
    sg = StreamGate("bf16", "bf16")
    v = np.array([0.0, 1e-45, 2.0 ** -126, 0.75, 1.0, 1.5, -3.0, 1e30, 2.0 ** -130])
    for dt in ("f32", "f16", "bf16"):
        sg.dtype = dt
        assert np.array_equal(sg._half_ulp(torch.from_numpy(v)).numpy(), half_ulp(v, dt))


def test_check_all_chains_plumbing(oracle_mod):
    """check_all_chains (the full-size GPU comparison) on host tensors: the oracle's own result
    rounded to the output dtypes passes; a copy with one head's y decayed wrongly by 1 % fails,
    whichever head block holds it."""
    from gpu_common import check_all_chains
    from mamba_ssd_prefill_amd.inputs import make_inputs
    inp = make_inputs(2, 150, 6, 16, 32, 2, dtype="bf16", state_dtype="f32", has_h0=True, seed=11)
    yr, fr = oracle_mod.recurrence_full(**inp.args())
    y = torch.from_numpy(yr).to(torch.bfloat16)
    fin = torch.from_numpy(fr).to(torch.float32)
    for hb in (0, 4):
        check_all_chains(inp, y, fin, "plumbing", heads_per_block=hb)
    core = torch.from_numpy(yr) - inp.x.double() * inp.D.double()[None, None, :, None]
    bad = torch.from_numpy(yr).clone()
    bad[1, :, 5] -= 0.02 * core[1, :, 5].abs().max()  # 2 % of the SSM term's scale on one head
    with pytest.raises(ParityError):
        check_all_chains(inp, bad.to(torch.bfloat16), fin, "plumbing", heads_per_block=4)
