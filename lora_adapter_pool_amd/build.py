"""Build liblora_pool.so (the C-ABI library) in-tree with hipcc for gfx950, and
the CPython binding of its per-call entry points (_lora_call) with gcc.

Usage: python -m lora_adapter_pool_amd.build   (or build_library() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import sysconfig
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblora_pool.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["lora_host.cpp", "lora_kernels.hip", "lora_meta.hip", "lora_merge.hip", "lora_api.hip"]
ARCH = os.environ.get("LORA_POOL_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
            "-Wno-unused-result"]


def device_flags():
    # packed fp32 VALU forms stay off: every fp32 op is a plain scalar instruction
    return [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops"]


def build_library(verbose: bool = False, jobs: int = 3) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="lora_pool_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            path = os.path.join(CSRC, src)
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc] + common_flags()
            if src.endswith(".hip"):
                cmd += ["-x", "hip"] + device_flags()
            cmd += ["-c", path, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            noise = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
            if p.returncode != 0:
                failed.append((src, "\n".join(noise)))
            elif verbose and noise:
                print("\n".join(noise))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(f"[{s}]\n{o}" for s, o in failed))
        out_tmp = os.path.join(tmp, LIB_NAME)
        link = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", out_tmp] + objs
        if verbose:
            print(" ".join(link), flush=True)
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(out_tmp, LIB_PATH)
        build_pycall(verbose)
        return LIB_PATH
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


PYCALL_SRC = os.path.join(CSRC, "lora_pycall.c")


def pycall_path() -> str:
    return os.path.join(PKG_DIR, "_lora_call" + sysconfig.get_config_var("EXT_SUFFIX"))


def build_pycall(verbose: bool = False) -> str:
    """The CPython binding of the per-call entry points (host code, gcc)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("gcc not found")
    out = pycall_path()
    tmp = out + ".tmp"
    cmd = [cc, "-O2", "-std=gnu11", "-shared", "-fPIC", "-Wall", "-Werror",
           f"-I{sysconfig.get_paths()['include']}", f"-I{INCLUDE}", PYCALL_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n" + r.stdout)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
