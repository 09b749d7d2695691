"""Builds libmkv.so in this package directory with hipcc for gfx950.

The library links against the HIP runtime that ships with the installed torch, so that a process that imports
torch and then loads libmkv.so holds a single HIP runtime (device pointers and streams are shared).
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmkv.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("MKV_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def torch_lib_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("torch is not importable: its HIP runtime is needed to link libmkv.so")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = []
    for f in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, f)
        obj = os.path.join(BUILD_DIR, f + ".o")
        if f.endswith(".hip"):
            jobs.append([hipcc, "-c", *HIP_FLAGS, src, "-o", obj])
        elif f.endswith(".cpp"):
            jobs.append([hipcc, "-c", *HOST_FLAGS, src, "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [j[-1] for j in jobs]
    tl = torch_lib_dir()
    tmp = LIB + ".tmp"
    _run(["g++", "-shared", "-o", tmp, *objs, f"-L{tl}", "-lamdhip64", f"-Wl,-rpath,{tl}", "-Wl,--no-undefined"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
