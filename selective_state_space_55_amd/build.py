"""Builds lib/libmamba_scan.so from csrc/*.hip with hipcc for gfx950.

Usage: python -m selective_state_space_55_amd.build  (or __graft_entry__.build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmamba_scan.so")
SOURCES = ["api.hip", "scan_fwd.hip", "scan_fwd_varlen.hip", "scan_step.hip", "scan_bwd.hip", "conv1d.hip", "ssd_fwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # packed fp32 VALU ops are kept out of generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err:
        print(err, file=sys.stderr)


# AddressSanitizer + UndefinedBehaviorSanitizer on the host code only (argument
# validation, planning, launches); the gfx950 code is built as usual.  The
# sanitizer runtime is not linked in: a process that loads this build preloads
# clang's libclang_rt.asan (see asan_runtime()).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime that matches hipcc's host compiler."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


def build(verbose: bool = False, out_path: str = LIB_PATH, host_sanitize: bool = False, defines=()) -> str:
    """Compiles each source to an object in parallel, then links the shared library.

    out_path, host_sanitize and defines make other builds of the same sources
    (the default is the library the package loads): host_sanitize adds
    HOST_SANITIZE, defines adds -D flags (MSCAN_LDS_POISON: every kernel fills
    its LDS with NaN before first use, so a read of a word no thread has
    written yet shows up in the results)."""
    from concurrent.futures import ThreadPoolExecutor

    out_dir = os.path.dirname(os.path.abspath(out_path))
    os.makedirs(out_dir, exist_ok=True)
    tag = os.path.splitext(os.path.basename(out_path))[0]
    obj_dir = os.path.join(LIB_DIR, "obj") if out_path == LIB_PATH else os.path.join(out_dir, "obj_" + tag)
    os.makedirs(obj_dir, exist_ok=True)
    extra = (HOST_SANITIZE if host_sanitize else []) + [f"-D{d}" for d in defines]
    cflags = [f for f in flags() if f != "-shared"] + extra
    objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc()] + cflags + ["-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out_path + ".tmp"
    link_extra = HOST_SANITIZE if host_sanitize else []
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + link_extra + objs, verbose)
    os.replace(tmp, out_path)
    return out_path


def asm(out_path: str) -> str:
    """Writes the gfx950 assembly of the kernels (for inspection)."""
    cmd = [hipcc()] + [f for f in flags() if f not in ("-shared", "-fPIC")] + [
        "--cuda-device-only", "-S", "-o", out_path, os.path.join(CSRC, "scan_fwd.hip")]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
