"""Builds ``librgdr.so`` (the gfx950 HIP library behind ``include/rgdr.h``) in-tree.

    python -m gated_delta_rule_rgdr_amd.build [--verbose]

Every source is compiled for gfx950 only. Packed fp32 instructions are switched off for
device code (``-target-feature -packed-fp32-ops``); the host pass prints a harmless
warning that it does not know that feature.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librgdr.so")

SOURCES = ["rgdr_decode.hip", "rgdr_prefill.hip", "la_gate.hip", "rgdr_host.cpp"]
ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def compile_cmd(src, obj, extra=()):
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    return (["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall"]
            + DEVICE_FLAGS + ["-I", INCLUDE, "-I", CSRC] + lang + list(extra)
            + ["-c", src, "-o", obj])


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o")
        cmd = compile_cmd(src, obj, extra)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for s, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass's note about the device-only feature is expected noise
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(s)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    link = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
