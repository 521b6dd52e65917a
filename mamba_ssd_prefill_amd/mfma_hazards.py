"""Build-time check of the gfx950 code objects for MFMA results read too early.

A VALU, memory or MFMA instruction that reads (or overwrites) the result registers of an MFMA
must issue a number of wait states after it (the hardware does not interlock; the compiler
inserts s_nop).  On straight-line code the compiler gives 8 wait states after
v_mfma_f32_16x16x32_{bf16,f16} and 10 after v_mfma_f32_16x16x4_f32 before such a read
(an MFMA that accumulates onto exactly those registers is chained by the hardware and needs
none).  Across a uniform branch, though, it has left some reads on the branch's short side
only 3 wait states after the MFMA: the read then saw a stale accumulator element (wrong y
for one p column in four of a block).

This module disassembles the code objects of the built translation units (our own build,
with llvm-objdump) and walks every control-flow path from each MFMA to the first
instruction that reads or writes its destination registers, counting wait states
conservatively (1 per instruction, n + 1 for s_nop n).  The build fails if any path is shorter than the
straight-line figure above, naming the kernel and the two instructions.
"""
import concurrent.futures
import os
import re
import subprocess
import tempfile

LLVM = os.environ.get("ROCM_LLVM", "/opt/rocm/llvm/bin")

# wait states between an MFMA and a dependent read, as the compiler inserts them on
# straight-line code for this target
REQUIRED = {
    "v_mfma_f32_16x16x32_bf16": 8,
    "v_mfma_f32_16x16x32_f16": 8,
    "v_mfma_f32_16x16x4_f32": 10,
}

_RANGE = re.compile(r"\b([av])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"\b([av])(\d+)\b")
_STORES = ("buffer_store", "global_store", "ds_write", "flat_store", "scratch_store")
_MEMORY = ("buffer_", "global_", "ds_", "flat_", "scratch_")


def _regs(text):
    out = set()
    for m in _RANGE.finditer(text):
        for r in range(int(m.group(2)), int(m.group(3)) + 1):
            out.add((m.group(1), r))
    for m in _SINGLE.finditer(_RANGE.sub("", text)):
        out.add((m.group(1), int(m.group(2))))
    return out


def _operands(args):
    return [p.strip() for p in args.split(",")] if args else []


def parse(text):
    """llvm-objdump -d --symbolize-operands output -> {kernel: (instructions, labels)};
    an instruction is (opcode, operand text)."""
    funcs, cur = {}, None
    for ln in text.splitlines():
        m = re.match(r"^<([^>]+)>:$", ln)
        if m:
            name = m.group(1)
            if re.match(r"^L\d+$", name):
                if cur is not None:
                    cur[1][name] = len(cur[0])
            else:
                cur = ([], {})
                funcs[name] = cur
            continue
        m = re.match(r"^\t([a-z][a-z0-9_]*)\s*(.*?)\s*(//.*)?$", ln)
        if m and cur is not None:
            cur[0].append((m.group(1), m.group(2)))
    return funcs


def short_paths(ins, labels):
    """Every (distance, required, mfma index, index of the instruction that reads or writes the
    MFMA's result registers) with a path shorter than required."""
    n = len(ins)
    succ = [[] for _ in range(n)]
    for i, (op, args) in enumerate(ins):
        tgt = args.split()[0] if args else ""
        if op == "s_branch":
            succ[i].append(labels[tgt])
        elif op.startswith("s_cbranch"):
            succ[i].append(labels[tgt])
            if i + 1 < n:
                succ[i].append(i + 1)
        elif op in ("s_endpgm", "s_setpc_b64", "s_trap"):
            pass
        elif i + 1 < n:
            succ[i].append(i + 1)
    found = []
    for k, (op, args) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        if op not in REQUIRED:
            raise ValueError("no wait-state figure for %s" % op)
        req = REQUIRED[op]
        dst0 = frozenset(_regs(_operands(args)[0]))
        best = {}
        stack = [(j, 0, dst0) for j in succ[k]]
        while stack:
            j, d, dst = stack.pop()
            if d >= req or best.get((j, dst), req) <= d:
                continue
            best[(j, dst)] = d
            op2, a2 = ins[j]
            o2 = _operands(a2)
            if op2.startswith("s_"):
                step = int(a2, 0) + 1 if op2 == "s_nop" else 1
                stack.extend((s_, d + step, dst) for s_ in succ[j])
                continue
            if op2.startswith("v_mfma"):
                ab = _regs(o2[1]) | _regs(o2[2])
                c = frozenset(_regs(o2[3])) if len(o2) > 3 else frozenset()
                # accumulating onto exactly these registers (C = the earlier result) is chained
                # by the hardware; as an A/B operand or in part of C they are a read
                if ab & dst or (c & dst and c != dst):
                    found.append((d, req, k, j))
                    continue
                dst = dst - _regs(o2[0])  # registers this MFMA writes now hold its result
                if not dst:
                    continue
            else:
                # a read; or a VALU overwrite before the result has landed (a load's data comes
                # back long after it issues, so only its address operands count)
                mem = op2.startswith(_MEMORY)
                touched = _regs(",".join(o2[1:] if mem and not op2.startswith(_STORES) else o2))
                if touched & dst:
                    found.append((d, req, k, j))
                    continue
            stack.extend((s_, d + 1, dst) for s_ in succ[j])
    return found


def has_device_code(obj):
    out = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-S", "--wide", obj],
                         check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
    return b".hip_fatbin" in out.stdout


def disassemble(obj):
    """The gfx950 code object of one compiled translation unit, disassembled."""
    with tempfile.TemporaryDirectory() as d:
        fb, co = os.path.join(d, "fb.bin"), os.path.join(d, "k.co")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section=.hip_fatbin=" + fb, obj],
                       check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + fb,
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--output=" + co],
                       check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--symbolize-operands",
                              "--no-show-raw-insn", "--no-leading-addr", co],
                             check=True, stdout=subprocess.PIPE, stderr=subprocess.PIPE)
    return out.stdout.decode()


def check_text(text):
    """Violations in one disassembly: list of readable lines."""
    bad = []
    for name, (ins, labels) in parse(text).items():
        for d, req, k, j in short_paths(ins, labels):
            bad.append("%s: %s -> %s %s after %d wait states (needs %d)"
                       % (name, ins[k][0], ins[j][0], ins[j][1][:40], d, req))
    return bad


def _check_object(obj):
    if not obj.endswith(".hip.o") or not has_device_code(obj):
        return []
    return ["%s: %s" % (os.path.basename(obj), b) for b in check_text(disassemble(obj))]


def check_objects(objs, workers=None):
    """Check the device code of every object that has any (in parallel processes); returns
    the violations."""
    workers = workers or min(8, os.cpu_count() or 1)
    with concurrent.futures.ProcessPoolExecutor(max_workers=workers) as ex:
        return [b for part in ex.map(_check_object, list(objs)) for b in part]
