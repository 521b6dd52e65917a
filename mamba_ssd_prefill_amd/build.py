"""Build libmamba_ssd.so in-tree with hipcc for gfx950.

    python -m mamba_ssd_prefill_amd.build

Each translation unit is compiled in its own hipcc process (in parallel), then linked.
"""
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmamba_ssd.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = (["ssd_api.cpp", "ssd_noalloc.hip", "ssd_common.hip", "ssd_decode.hip", "ssd_block.hip", "ssd_kernels_f32.hip", "ssd_kernels_f32_vl.hip",
            "ssd_kernels_f16.hip", "ssd_kernels_bf16.hip", "ssd_kernels_f16_blk.hip", "ssd_kernels_bf16_blk.hip"]
           + ["ssd_kernels_%s_q%d%s.hip" % (d, q, v) for d in ("f16", "bf16") for q in (64, 128, 256)
              for v in ("", "_vl")])

ARCH = os.environ.get("MAMBA_SSD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 (v_pk_*_f32) instructions.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(force=True, verbose=False):
    """Compile every HIP translation unit and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        path = os.path.join(CSRC, src)
        if not force and os.path.exists(obj) and os.path.getmtime(obj) >= _newest_input(path):
            continue
        cmd = [HIPCC] + CFLAGS + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines() if "packed-fp32-ops" not in l)
        if pr.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join("== %s ==\n%s" % f for f in failed))
    # MFMA results read too early on some control-flow path (a compiler hazard gap): fail here
    from . import mfma_hazards
    bad = mfma_hazards.check_objects(objs)
    if bad:
        raise RuntimeError("MFMA results read too early:\n" + "\n".join(bad[:40]))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, LIB)
    return LIB


def source_hash():
    """Short hash of every kernel source file (csrc/ and the C header): a profile taken on
    other sources is stale."""
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _newest_input(src):
    t = os.path.getmtime(src)
    for f in os.listdir(CSRC):
        if f.endswith(".h"):
            t = max(t, os.path.getmtime(os.path.join(CSRC, f)))
    t = max(t, os.path.getmtime(os.path.join(ROOT, "include", "mamba_ssd.h")))
    return t


if __name__ == "__main__":
    print(build(force="--incremental" not in sys.argv, verbose=True))
