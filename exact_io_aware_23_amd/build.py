"""Compile the HIP sources into the in-tree shared library libattn.so (gfx950).

Run `python -m exact_io_aware_23_amd.build` or call build().  Always compiles;
hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
SOURCES = ["attn_api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_fwd_fp8.hip", "attn_probe.hip"]
# per-file extra flags (none at present)
EXTRA_FLAGS: dict = {}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # no packed fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, out: str | None = None, build_dir: str | None = None,
          defines: tuple = ()) -> str:
    """Compile every source and link the library (to `out`, default libattn.so)."""
    bdir = build_dir or BUILD_DIR
    lib_path = out or LIB_PATH
    os.makedirs(bdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), *defines, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
        if p.returncode != 0:
            failed.append((src, out))
        elif text and verbose:
            print(text, flush=True)
    if failed:
        for src, out in failed:
            sys.stderr.write(f"hipcc failed for {src}:\n{out}\n")
        raise RuntimeError("HIP build failed: " + ", ".join(s for s, _ in failed))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
