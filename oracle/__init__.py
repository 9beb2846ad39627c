"""fp64 CPU oracle for the selective scan (forward pass, single-token step, backward pass) and
the causal conv1d + SiLU in front of it.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, links or executes anything
here, and nothing here imports the product package.

The arithmetic lives in ``scan_oracle.c`` (plain C, double precision, one
sequential time loop per (batch, channel); see its header for the passages of
the pages each step follows).  This module only builds that file with gcc,
loads it with ctypes and converts arguments to contiguous float64 arrays.
Inputs given in bfloat16 or float32 are widened exactly (every bf16/fp32
value is representable in fp64), so the oracle sees the very values the GPU
consumes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "scan_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_scan.so")
_lib = None


def build(verbose: bool = False, out_path: str = _LIB_PATH, sanitize: bool = False) -> str:
    """Compile scan_oracle.c with gcc (-O2, no fast-math, OpenMP).  sanitize: clang
    with AddressSanitizer + UndefinedBehaviorSanitizer instead (clang's OpenMP
    runtime; no sanitizer runtime linked in: the process preloads clang's)."""
    if sanitize:
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               "-Wl,-rpath,/opt/rocm/llvm/lib", "-o", out_path + ".tmp", _SRC, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", out_path + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_scan_fwd.restype = ctypes.c_int
    lib.oracle_scan_fwd.argtypes = [P] * 11 + [I64] * 4 + [ctypes.c_int] * 3
    lib.oracle_scan_step.restype = ctypes.c_int
    lib.oracle_scan_fwd_varlen.restype = ctypes.c_int
    lib.oracle_scan_fwd_varlen.argtypes = [P] * 12 + [I64] * 4 + [ctypes.c_int] * 3
    lib.oracle_ssd_fwd.restype = ctypes.c_int
    lib.oracle_ssd_fwd.argtypes = [P] * 11 + [I64] * 5 + [ctypes.c_int] * 3
    lib.oracle_scan_step.argtypes = [P] * 9 + [ctypes.c_int, ctypes.c_int, P] + [I64] * 3 + [ctypes.c_int]
    lib.oracle_scan_bwd.restype = ctypes.c_int
    lib.oracle_scan_bwd.argtypes = [P] * 20 + [I64] * 4 + [ctypes.c_int] * 3
    lib.oracle_conv1d_fwd.restype = ctypes.c_int
    lib.oracle_conv1d_fwd.argtypes = [P] * 6 + [I64] * 4 + [ctypes.c_int, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    other = os.environ.get("ORACLE_SCAN_LIBRARY")   # another build (a sanitizer build)
    if other:
        _lib = _bind(other)
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(_LIB_PATH)
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(a, shape=None) -> Optional[np.ndarray]:
    """Exact widening to a C-contiguous float64 array (accepts numpy or torch CPU)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        import torch

        a = a.detach().to("cpu")
        if a.dtype in (torch.bfloat16, torch.float16):
            a = a.to(torch.float32)
        a = a.numpy()
    out = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and out.shape != tuple(shape):
        raise ValueError(f"oracle: expected shape {tuple(shape)}, got {out.shape}")
    return out


def _euler(discretization: str) -> int:
    if discretization not in ("zoh", "euler"):
        raise ValueError(f"oracle: discretization must be 'zoh' or 'euler', got {discretization!r}")
    return int(discretization == "euler")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan_fwd(u, delta, A_log, B, C, D=None, z=None, delta_bias=None, initial_state=None,
             delta_softplus: bool = True, return_final_state: bool = True,
             nthreads: int = 0, _lib_override=None, discretization: str = "zoh"
             ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Selective-scan forward in fp64 (discretization "zoh", or "euler": Bbar = Delta B).

    Shapes: u, delta, z: (batch, dim, L); B, C: (batch, dstate, L); A_log: (dim, dstate);
    D, delta_bias: (dim,); initial_state: (batch, dim, dstate).
    Returns (y (batch, dim, L) float64, final_state (batch, dim, dstate) float64 or None).
    """
    u = _f64(u)
    if u.ndim != 3:
        raise ValueError("oracle: u must be (batch, dim, L)")
    batch, dim, L = u.shape
    A_log = _f64(A_log)
    dstate = A_log.shape[1]
    delta = _f64(delta, (batch, dim, L))
    A_log = _f64(A_log, (dim, dstate))
    B = _f64(B, (batch, dstate, L))
    C = _f64(C, (batch, dstate, L))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim, L))
    delta_bias = _f64(delta_bias, (dim,))
    initial_state = _f64(initial_state, (batch, dim, dstate))
    y = np.empty((batch, dim, L), dtype=np.float64)
    fs = np.empty((batch, dim, dstate), dtype=np.float64) if return_final_state else None
    rc = (_lib_override or _load()).oracle_scan_fwd(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                 _ptr(delta_bias), _ptr(initial_state), _ptr(fs), _ptr(y), batch, dim,
                                 dstate, L, int(bool(delta_softplus)), _euler(discretization), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_scan_fwd returned {rc}")
    return y, fs


def scan_fwd_varlen(u, delta, A_log, B, C, cu_seqlens, D=None, z=None, delta_bias=None, initial_states=None,
                    delta_softplus: bool = True, discretization: str = "zoh", nthreads: int = 0,
                    _lib_override=None) -> Tuple[np.ndarray, np.ndarray]:
    """Variable-length batch in fp64: nseq sequences packed along time, sequence s on tokens
    [cu_seqlens[s], cu_seqlens[s+1]).  u, delta, z: (dim, total); B, C: (dstate, total);
    initial_states: (nseq, dim, dstate).  Returns (y (dim, total), final_states (nseq, dim, dstate))."""
    u = _f64(u)
    if u.ndim != 2:
        raise ValueError("oracle: u must be (dim, total)")
    dim, total = u.shape
    A_log = _f64(A_log)
    dstate = A_log.shape[1]
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).ravel())
    nseq = cu.size - 1
    delta = _f64(delta, (dim, total))
    A_log = _f64(A_log, (dim, dstate))
    B = _f64(B, (dstate, total))
    C = _f64(C, (dstate, total))
    D = _f64(D, (dim,))
    z = _f64(z, (dim, total))
    delta_bias = _f64(delta_bias, (dim,))
    initial_states = _f64(initial_states, (nseq, dim, dstate))
    y = np.zeros((dim, total), dtype=np.float64)
    fs = np.empty((nseq, dim, dstate), dtype=np.float64)
    rc = (_lib_override or _load()).oracle_scan_fwd_varlen(
        _ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(cu),
        _ptr(initial_states), _ptr(fs), _ptr(y), nseq, dim, dstate, total, int(bool(delta_softplus)),
        _euler(discretization), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_scan_fwd_varlen returned {rc}")
    return y, fs


def ssd_fwd(x, dt, A_log, B, C, D=None, z=None, dt_bias=None, initial_state=None, dt_softplus: bool = True,
            discretization: str = "zoh", nthreads: int = 0, _lib_override=None) -> Tuple[np.ndarray, np.ndarray]:
    """Multi-head SSM with a scalar decay per head, fp64.  x, z: (batch, L, H, P); dt: (batch, L, H);
    B, C: (batch, L, N); A_log, D, dt_bias: (H,); initial_state: (batch, H, P, N).
    Returns (y (batch, L, H, P), final_state (batch, H, P, N))."""
    x = _f64(x)
    if x.ndim != 4:
        raise ValueError("oracle: x must be (batch, L, H, P)")
    batch, L, H, P = x.shape
    B = _f64(B)
    N = B.shape[-1]
    dt = _f64(dt, (batch, L, H))
    A_log = _f64(A_log, (H,))
    B = _f64(B, (batch, L, N))
    C = _f64(C, (batch, L, N))
    D = _f64(D, (H,))
    z = _f64(z, (batch, L, H, P))
    dt_bias = _f64(dt_bias, (H,))
    initial_state = _f64(initial_state, (batch, H, P, N))
    y = np.empty((batch, L, H, P), dtype=np.float64)
    fs = np.empty((batch, H, P, N), dtype=np.float64)
    rc = (_lib_override or _load()).oracle_ssd_fwd(
        _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(initial_state),
        _ptr(fs), _ptr(y), batch, L, H, P, N, int(bool(dt_softplus)), _euler(discretization), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_ssd_fwd returned {rc}")
    return y, fs


def scan_step(state, x, dt, A_log, B, C, D=None, z=None, dt_bias=None, dt_softplus: bool = True,
              nthreads: int = 0, _lib_override=None, discretization: str = "zoh") -> Tuple[np.ndarray, np.ndarray]:
    """One recurrent step in fp64.  Returns (y (batch, dim), new_state (batch, dim, dstate)).

    Shapes: state: (batch, dim, dstate); x, dt, z: (batch, dim); B, C: (batch, dstate);
    A_log: (dim, dstate); D, dt_bias: (dim,).  The input state is not modified.
    """
    st = _f64(state).copy()
    if st.ndim != 3:
        raise ValueError("oracle: state must be (batch, dim, dstate)")
    batch, dim, dstate = st.shape
    x = _f64(x, (batch, dim))
    dt = _f64(dt, (batch, dim))
    A_log = _f64(A_log, (dim, dstate))
    B = _f64(B, (batch, dstate))
    C = _f64(C, (batch, dstate))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim))
    dt_bias = _f64(dt_bias, (dim,))
    y = np.empty((batch, dim), dtype=np.float64)
    rc = (_lib_override or _load()).oracle_scan_step(_ptr(st), _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                  _ptr(z), _ptr(dt_bias), int(bool(dt_softplus)), _euler(discretization), _ptr(y),
                                  batch, dim,
                                  dstate, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_scan_step returned {rc}")
    return y, st


def scan_bwd(u, delta, A_log, B, C, dy, D=None, z=None, delta_bias=None, initial_state=None,
             d_final_state=None, delta_softplus: bool = True, nthreads: int = 0, _lib_override=None,
             discretization: str = "zoh") -> dict:
    """Gradients of the selective-scan forward in fp64 (discretization "zoh", or "euler" for
    Bbar u = Delta B u), given dL/dy (and optionally dL/d final_state).  Returns a dict with du, ddelta, dA_log, dB, dC (always) and dD,
    dz, ddelta_bias, d_initial_state (when D, z, delta_bias, initial_state are given)."""
    u = _f64(u)
    if u.ndim != 3:
        raise ValueError("oracle: u must be (batch, dim, L)")
    batch, dim, L = u.shape
    A_log = _f64(A_log)
    dstate = A_log.shape[1]
    delta = _f64(delta, (batch, dim, L))
    B = _f64(B, (batch, dstate, L))
    C = _f64(C, (batch, dstate, L))
    dy = _f64(dy, (batch, dim, L))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim, L))
    delta_bias = _f64(delta_bias, (dim,))
    initial_state = _f64(initial_state, (batch, dim, dstate))
    d_final_state = _f64(d_final_state, (batch, dim, dstate))
    g = {"du": np.empty((batch, dim, L)), "ddelta": np.empty((batch, dim, L)), "dA_log": np.empty((dim, dstate)),
         "dB": np.empty((batch, dstate, L)), "dC": np.empty((batch, dstate, L))}
    g["dD"] = np.empty((dim,)) if D is not None else None
    g["dz"] = np.empty((batch, dim, L)) if z is not None else None
    g["ddelta_bias"] = np.empty((dim,)) if delta_bias is not None else None
    g["d_initial_state"] = np.empty((batch, dim, dstate)) if initial_state is not None else None
    rc = (_lib_override or _load()).oracle_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        _ptr(initial_state), _ptr(dy), _ptr(d_final_state), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA_log"]),
        _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddelta_bias"]),
        _ptr(g["d_initial_state"]), batch, dim, dstate, L, int(bool(delta_softplus)), _euler(discretization),
        int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_scan_bwd returned {rc}")
    return g


def conv1d_fwd(x, weight, bias=None, conv_state=None, silu: bool = True, return_state: bool = False,
               nthreads: int = 0, _lib_override=None):
    """Causal depthwise conv1d (+ SiLU) in fp64.  x: (batch, dim, L); weight: (dim, K); bias: (dim,);
    conv_state: (batch, dim, K-1), oldest first.  Returns u (batch, dim, L) [, final conv state]."""
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("oracle: x must be (batch, dim, L)")
    batch, dim, L = x.shape
    weight = _f64(weight)
    K = weight.shape[1]
    weight = _f64(weight, (dim, K))
    bias = _f64(bias, (dim,))
    conv_state = _f64(conv_state, (batch, dim, K - 1))
    u = np.empty((batch, dim, L))
    st = np.empty((batch, dim, K - 1)) if return_state else None
    rc = (_lib_override or _load()).oracle_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state), _ptr(st),
                                                      _ptr(u), batch, dim, L, K, int(bool(silu)), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_conv1d_fwd returned {rc}")
    return (u, st) if return_state else u


class Variant:
    """The same wrapper bound to another build of scan_oracle.c (used by the
    tests that plant a mistake in a copy of the oracle and check that the pins
    catch it)."""

    def __init__(self, lib_path: str):
        self._lib = _bind(lib_path)

    def scan_fwd(self, *a, **k):
        return scan_fwd(*a, _lib_override=self._lib, **k)

    def scan_step(self, *a, **k):
        return scan_step(*a, _lib_override=self._lib, **k)

    def scan_fwd_varlen(self, *a, **k):
        return scan_fwd_varlen(*a, _lib_override=self._lib, **k)

    def ssd_fwd(self, *a, **k):
        return ssd_fwd(*a, _lib_override=self._lib, **k)

    def scan_bwd(self, *a, **k):
        return scan_bwd(*a, _lib_override=self._lib, **k)

    def conv1d_fwd(self, *a, **k):
        return conv1d_fwd(*a, _lib_override=self._lib, **k)


def build_variant(src_text: str, out_dir: str, name: str) -> "Variant":
    """Compile C source text (a modified copy of scan_oracle.c) and bind it."""
    src = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, "lib" + name + ".so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, src, "-lm"], check=True)
    return Variant(so)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
