"""C-ABI tests that run without a GPU.

The library must load, export every function include/mamba_ssd.h declares, and reject
bad arguments on the host before any HIP call.  Every call here fails exactly one check
with otherwise valid arguments (fake but aligned addresses), so no kernel is ever
launched -- these tests are safe on a GPU machine too.
"""
import ctypes
import os
import re

import pytest

import mamba_ssd_prefill_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba_ssd.h")

OK, NULLP, SHAPE, UNSUP, MISAL, WS_SMALL, HIP, TIMEOUT, BADARG, SCHEDULE = range(10)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return ssd.load_library()


def base(**kw):
    p = dict(batch=2, seqlen=300, nheads=8, headdim=64, dstate=128, ngroups=2, chunk_size=128,
             in_dtype="bf16", state_dtype="f32", dt_softplus=True, impl="fused")
    p.update(kw)
    return ssd.make_params(**p)


def test_header_and_binding_agree():
    assert header_functions() == sorted(ssd.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_function(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_abi_struct_sizes_match_header(tmp_path):
    """The binding's ctypes structs have the C header's sizes and field offsets (gcc, LP64)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    checks = [("ssd_params_t", ssd.Params), ("ssd_workspace_layout_t", ssd.Layout)]
    lines = []
    for cname, cls in checks:
        lines.append('    printf("%%s %%zu\\n", "%s", sizeof(%s));' % (cname, cname))
        for f, _ in cls._fields_:
            lines.append('    printf("%%s.%%s %%zu\\n", "%s", "%s", offsetof(%s, %s));' % (cname, f, cname, f))
    src = tmp_path / "sizes.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mamba_ssd.h"\nint main(void) {\n%s\n'
                   "    return 0;\n}\n" % "\n".join(lines))
    exe = tmp_path / "sizes"
    r = subprocess.run([gcc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    for cname, cls in checks:
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got["%s.%s" % (cname, f)]) == getattr(cls, f).offset, (cname, f)


def test_status_strings(lib):
    for code in range(11):
        s = lib.ssd_status_string(code)
        assert s and len(s) > 3
    assert lib.ssd_status_string(1234) == b"unknown status"


@pytest.mark.parametrize("kw,code", [
    (dict(), OK),
    (dict(batch=0), SHAPE), (dict(seqlen=0), SHAPE), (dict(nheads=0), SHAPE),
    (dict(ngroups=3), SHAPE), (dict(ngroups=0), SHAPE), (dict(chunk_size=0), SHAPE),
    (dict(headdim=48), UNSUP), (dict(headdim=256), UNSUP), (dict(dstate=16), UNSUP),
    (dict(dstate=256), UNSUP), (dict(chunk_size=32), UNSUP), (dict(chunk_size=100), UNSUP),
    (dict(chunk_size=512), UNSUP),
    (dict(dstate=16, in_dtype="f32"), OK), (dict(chunk_size=192), UNSUP), (dict(headdim=128), OK),
    (dict(in_dtype=3), BADARG), (dict(state_dtype=-1), BADARG), (dict(impl=2), BADARG),
    (dict(dt_softplus=True, impl="unfused"), OK),
])
def test_validate(lib, kw, code):
    assert lib.ssd_validate(ctypes.byref(base(**kw))) == code


def test_validate_rejects_short_struct_and_null(lib):
    p = base()
    p.struct_size = 8
    assert lib.ssd_validate(ctypes.byref(p)) == BADARG
    assert lib.ssd_validate(None) == NULLP
    p = base()
    p.dt_softplus = 2
    assert lib.ssd_validate(ctypes.byref(p)) == BADARG


def test_params_abi_version_1_and_relaxed_field(lib):
    """A caller built against ABI version 1 passes the struct size that ends before `relaxed`
    (56 bytes on LP64): accepted, with relaxed = 0 whatever the trailing bytes hold.  With the
    full struct, relaxed must be 0 or 1 and flags 0 or SSD_FLAG_WORKSPACE_READY; relaxed halves
    the CB region (16-bit inputs only)."""
    p = base()
    p.struct_size = ssd.Params.relaxed.offset
    p.relaxed, p.flags = 7, 9  # not read with the version-1 size
    assert lib.ssd_validate(ctypes.byref(p)) == OK
    p.struct_size = ssd.Params.relaxed.offset - 4
    assert lib.ssd_validate(ctypes.byref(p)) == BADARG
    q = base()
    q.relaxed = 2
    assert lib.ssd_validate(ctypes.byref(q)) == BADARG
    q = base()
    q.flags = ssd.FLAG_WORKSPACE_READY
    assert lib.ssd_validate(ctypes.byref(q)) == OK
    assert ssd.workspace_size(q) == ssd.workspace_size(base())  # the flag changes no size
    for bad in (2, 4, -1):
        q.flags = bad
        assert lib.ssd_validate(ctypes.byref(q)) == BADARG
    for impl in ("fused", "unfused"):
        exact = ssd.workspace_layout(base(impl=impl))
        rel = ssd.workspace_layout(base(impl=impl, relaxed=True))
        assert rel.cb_bytes * 2 == exact.cb_bytes
        f32 = ssd.workspace_layout(base(impl=impl, in_dtype="f32", relaxed=True))
        assert f32.cb_bytes == ssd.workspace_layout(base(impl=impl, in_dtype="f32")).cb_bytes


def test_validate_rejects_ticket_overflow(lib):
    p = base(batch=4096, seqlen=1 << 20, nheads=128, ngroups=128, chunk_size=64)
    assert lib.ssd_validate(ctypes.byref(p)) == SHAPE


@pytest.mark.parametrize("impl", ["fused", "unfused"])
@pytest.mark.parametrize("state", ["f32", "f16"])
@pytest.mark.parametrize("relay", ["0", "1", ""])
def test_workspace_layout_arithmetic(lib, impl, state, relay, monkeypatch):
    monkeypatch.setenv("MAMBA_SSD_RELAY", relay)
    p = base(impl=impl, state_dtype=state)
    lay = ssd.workspace_layout(p)
    Bt, L, H, P, N, G, Q = 2, 300, 8, 64, 128, 2, 128
    nc = -(-L // Q)
    es = 4 if state == "f32" else 2
    fused = impl == "fused"
    # the relay form's buffers: forced on or off, else by shape (8 chains here: on)
    relay_ws = fused and relay != "0"
    assert lay.nchunks == nc
    K = (2 if relay_ws else 1) if fused else nc + 1
    assert lay.state_slots == K
    assert lay.dt_bytes == Bt * nc * H * Q * 4 == lay.acs_bytes
    # fused: one CB run per (partition, (b, g) pair); at most B*G + 7 with up to 8 partitions
    pair_slots = Bt * G + 7
    assert lay.cb_bytes == (pair_slots if fused else Bt * G) * nc * Q * Q * 4
    # fused relay form: a 10-slot chunk-state ring (fp32; fp16 with fp16 state storage) and a
    # min(6, nc + 1)-slot operand ring (input dtype, bf16 here) per chain
    relay_bytes = Bt * H * P * N * ((2 if state == "f16" else 4) * 10 + 2 * min(6, nc + 1))
    assert lay.s_bytes == ((relay_bytes if relay_ws else 0) if fused else Bt * nc * H * P * N * 4)
    assert lay.states_bytes == Bt * K * H * P * N * es
    assert lay.seg_bytes == Bt * nc * Q * 4
    regions = sorted([(lay.dt_offset, lay.dt_bytes), (lay.acs_offset, lay.acs_bytes), (lay.cb_offset, lay.cb_bytes),
                      (lay.s_offset, lay.s_bytes), (lay.states_offset, lay.states_bytes),
                      (lay.seg_offset, lay.seg_bytes), (lay.sync_offset, lay.sync_bytes)])
    for (o1, n1), (o2, _) in zip(regions, regions[1:]):
        assert o1 % 256 == 0 and o1 + n1 <= o2
    assert lay.sync_offset <= lay.status_offset < lay.sync_offset + lay.sync_bytes
    assert lay.total_bytes >= lay.sync_offset + lay.sync_bytes
    assert ssd.workspace_size(p) == lay.total_bytes
    if fused:
        # per-chain words [B][H][P/32] (three 128-byte lines each), cs_done and bmm_done
        # [pair slots][nc], 8 partition tickets 32 words apart, 8 owner, 8 joined and 8 relay
        # decision words, exit counter, abort, status
        assert lay.sync_bytes == 4 * (Bt * H * 2 * 96 + 2 * pair_slots * nc + 8 * 32 + 24 + 3)
    else:
        assert lay.sync_bytes == 8  # abort and status words


def test_workspace_size_zero_for_invalid(lib):
    assert lib.ssd_prefill_workspace_size(ctypes.byref(base(headdim=48))) == 0
    assert lib.ssd_prefill_workspace_size(None) == 0


FAKE = 1 << 40  # an aligned address that is never dereferenced


def prefill_args(p, **over):
    ws = ssd.workspace_size(p)
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=FAKE, dt_bias=FAKE, h0=FAKE, y=FAKE, fin=FAKE,
             ws=FAKE, ws_bytes=ws, stream=None)
    a.update(over)
    return a


def call_prefill(lib, p, a):
    vp = ctypes.c_void_p
    return lib.ssd_prefill(ctypes.byref(p), vp(a["x"]), vp(a["dt"]), vp(a["A"]), vp(a["B"]), vp(a["C"]),
                           vp(a["D"]), vp(a["dt_bias"]), vp(a["h0"]), vp(a["y"]), vp(a["fin"]), vp(a["ws"]),
                           a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("field", ["x", "dt", "A", "B", "C", "y", "fin", "ws"])
def test_prefill_null_pointers(lib, field):
    p = base()
    assert call_prefill(lib, p, prefill_args(p, **{field: None})) == NULLP


@pytest.mark.parametrize("field,off", [("x", 8), ("B", 4), ("C", 2), ("y", 8), ("fin", 8), ("h0", 8),
                                       ("dt", 1), ("A", 2), ("D", 2), ("dt_bias", 2), ("ws", 128)])
def test_prefill_misaligned(lib, field, off):
    p = base()
    assert call_prefill(lib, p, prefill_args(p, **{field: FAKE + off})) == MISAL


def test_prefill_workspace_too_small(lib):
    p = base()
    assert call_prefill(lib, p, prefill_args(p, ws_bytes=ssd.workspace_size(p) - 1)) == WS_SMALL


def test_prefill_invalid_params(lib):
    p = base(headdim=48)
    assert call_prefill(lib, p, prefill_args(base(), ws_bytes=1 << 30)) == UNSUP
    p = base(ngroups=3)
    assert call_prefill(lib, p, prefill_args(base(), ws_bytes=1 << 30)) == SHAPE


def test_steps_require_unfused_params(lib):
    p = base(impl="fused")
    vp = ctypes.c_void_p
    ws = ssd.workspace_size(p)
    assert lib.ssd_step_bmm(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), ws, None) == BADARG
    assert lib.ssd_step_chunk_cumsum(ctypes.byref(p), vp(FAKE), vp(FAKE), None, vp(FAKE), ws, None) == BADARG


def test_steps_validate_before_launch(lib):
    p = base(impl="unfused")
    vp = ctypes.c_void_p
    ws = ssd.workspace_size(p)
    assert lib.ssd_step_bmm(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), ws - 1, None) == WS_SMALL
    assert lib.ssd_step_bmm(ctypes.byref(p), None, vp(FAKE), vp(FAKE), ws, None) == NULLP
    assert lib.ssd_step_chunk_state(ctypes.byref(p), vp(FAKE + 2), vp(FAKE), vp(FAKE), ws, None) == MISAL
    assert lib.ssd_step_chunk_scan(ctypes.byref(p), vp(FAKE), vp(FAKE), None, None, vp(FAKE), ws, None) == NULLP
    assert lib.ssd_step_state_passing(ctypes.byref(p), None, None, vp(FAKE), ws, None) == NULLP
    assert lib.ssd_step_chunk_cumsum(ctypes.byref(p), vp(FAKE + 1), vp(FAKE), None, vp(FAKE), ws, None) == MISAL


def test_check_device_status_validates_first(lib):
    assert lib.ssd_check_device_status(ctypes.byref(base(headdim=48)), ctypes.c_void_p(FAKE), None) == UNSUP
    assert lib.ssd_check_device_status(ctypes.byref(base()), None, None) == NULLP


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 64, 4, 16)
    B = torch.zeros(1, 64, 1, 16)
    with pytest.raises(ValueError):
        ssd.ssd_prefill(x, torch.zeros(1, 64, 4), torch.zeros(4), B, B.clone())


# ---- the decode step: host validation only (every call fails one check, nothing launches) -----
def dec_params(**kw):
    p = dict(batch=2, seqlen=1, nheads=8, headdim=64, dstate=128, ngroups=2, chunk_size=128,
             in_dtype="bf16", state_dtype="f32", dt_softplus=True, impl="fused")
    p.update(kw)
    return ssd.make_params(**p)


DEC_FIELDS = ["x", "dt", "A", "B", "C", "D", "dt_bias", "state_in", "state_out", "y"]


def dec_call(lib, prm, **override):
    ptrs = {f: 0x10000 * (i + 1) for i, f in enumerate(DEC_FIELDS)}
    ptrs.update(override)
    return lib.ssd_decode_step(ctypes.byref(prm), *[ptrs[f] for f in DEC_FIELDS], None)


@pytest.mark.parametrize("kw,code", [
    (dict(seqlen=2), SHAPE), (dict(seqlen=0), SHAPE), (dict(batch=0), SHAPE), (dict(nheads=0), SHAPE),
    (dict(headdim=0), SHAPE), (dict(ngroups=3), SHAPE), (dict(dstate=48), UNSUP), (dict(dstate=512), UNSUP),
    (dict(dstate=8), UNSUP), (dict(in_dtype=3), BADARG), (dict(state_dtype=5), BADARG),
])
def test_decode_rejects_bad_params(lib, kw, code):
    assert dec_call(lib, dec_params(**kw)) == code


@pytest.mark.parametrize("field", ["x", "dt", "A", "B", "C", "state_out", "y"])
def test_decode_null_pointers(lib, field):
    assert dec_call(lib, dec_params(), **{field: None}) == NULLP


@pytest.mark.parametrize("field,off", [("x", 8), ("B", 4), ("C", 2), ("y", 8), ("state_in", 8), ("state_out", 4),
                                       ("A", 2), ("D", 1), ("dt_bias", 2), ("dt", 1)])
def test_decode_misaligned(lib, field, off):
    assert dec_call(lib, dec_params(), **{field: 0x10000 * (DEC_FIELDS.index(field) + 1) + off}) == MISAL


def test_decode_short_struct(lib):
    p = dec_params()
    p.struct_size = 8
    assert dec_call(lib, p) == BADARG
    assert lib.ssd_decode_step(None, *([0x10000] * 10), None) == NULLP


# ---- packed variable-length prefill: host validation only ------------------------------------
def call_varlen(lib, p, a, seq):
    vp = ctypes.c_void_p
    return lib.ssd_prefill_varlen(ctypes.byref(p), vp(a["x"]), vp(a["dt"]), vp(a["A"]), vp(a["B"]), vp(a["C"]),
                                  vp(a["D"]), vp(a["dt_bias"]), vp(seq), vp(a["h0"]), vp(a["y"]), vp(a["fin"]),
                                  vp(a["ws"]), a["ws_bytes"], a["stream"])


def test_varlen_requires_aligned_seq_idx(lib):
    p = base()
    assert call_varlen(lib, p, prefill_args(p), None) == NULLP
    assert call_varlen(lib, p, prefill_args(p), FAKE + 2) == MISAL


@pytest.mark.parametrize("field", ["x", "C", "fin", "ws"])
def test_varlen_validates_like_prefill(lib, field):
    p = base()
    assert call_varlen(lib, p, prefill_args(p, **{field: None}), FAKE) == NULLP
    assert call_varlen(lib, base(headdim=48), prefill_args(p, ws_bytes=1 << 30), FAKE) == UNSUP
    assert call_varlen(lib, p, prefill_args(p, ws_bytes=ssd.workspace_size(p) - 1), FAKE) == WS_SMALL


def test_header_compiles_as_plain_c(tmp_path):
    """include/mamba_ssd.h is a C header: a C11 translation unit that takes the address of every
    declared function compiles with gcc (no HIP or C++ needed by callers)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use_header.c"
    refs = "\n".join("    (void)&%s;" % f for f in header_functions())
    src.write_text('#include "mamba_ssd.h"\nint main(void) {\n    ssd_params_t p = {0};\n    (void)p;\n%s\n'
                   "    return 0;\n}\n" % refs)
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                        str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_noalloc_refuses_a_problem_larger_than_the_scratch(lib):
    """ssd_prefill_noalloc checks the problem's workspace against its static scratch before any
    HIP call (so this runs without a GPU): the 262K-token context needs more than it holds."""
    prm = ssd.make_params(1, 262144, 80, 64, 128, 1, 128, "f16", "f16", True, "fused")
    assert ssd.workspace_size(prm) > (320 << 20)
    fake = ctypes.c_void_p(FAKE)
    rc = lib.ssd_prefill_noalloc(ctypes.byref(prm), fake, fake, fake, fake, fake, None, None, None, fake, fake, None)
    assert ssd.STATUS_NAMES[rc] == "SSD_ERR_SCRATCH_TOO_SMALL"
    assert lib.ssd_prefill_noalloc(ctypes.byref(base(headdim=48)), fake, fake, fake, fake, fake, None, None, None,
                                   fake, fake, None) == UNSUP


def test_varlen_states_validates_before_launch(lib):
    """ssd_prefill_varlen_states refuses fp32 inputs, nseq < 1 and missing or misaligned state
    arrays before any HIP call (fake pointers, no GPU needed)."""
    p = base()
    f = ctypes.c_void_p(FAKE)

    def call(prm, nseq=3, seq=FAKE, h0=FAKE, fin=FAKE):
        return lib.ssd_prefill_varlen_states(ctypes.byref(prm), f, f, f, f, f, None, None, ctypes.c_void_p(seq) if seq else None,
                                             nseq, ctypes.c_void_p(h0) if h0 else None, f,
                                             ctypes.c_void_p(fin) if fin else None, f, ssd.workspace_size(prm), None)
    assert call(base(in_dtype="f32")) == UNSUP
    assert call(p, nseq=0) == SHAPE
    assert call(p, fin=0) == NULLP
    assert call(p, seq=0) == NULLP
    assert call(p, h0=FAKE + 8) == MISAL
    assert call(p, fin=FAKE + 8) == MISAL
