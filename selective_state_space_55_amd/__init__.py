"""MI355X-native selective scan (Mamba): Python binding over libmamba_scan.so.

This module only marshals arguments: it checks torch tensors (device, dtype,
contiguity, shape), allocates outputs and the workspace with torch, and calls
the C ABI declared in include/mamba_scan.h.  Every step of the computation
runs in the library's HIP kernels.  If the library is not built, importing
works but every call raises; there is no fallback.

Streams: each call runs on its `stream` argument (a torch stream or a raw HIP
stream handle), or on the current stream when it is None.  Outputs and the
workspace a call allocates are allocated while that stream is current, so
torch's caching allocator hands their memory to no other stream's work before
the kernels are done with it.  Tensors the caller passes in (inputs, `out=`,
`workspace=`) are the caller's to keep alive and ordered with that stream.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MAMBA_SCAN_LIBRARY names another build of the same library (a sanitizer or
# debug build); by default the in-tree build is loaded
LIB_PATH = os.environ.get("MAMBA_SCAN_LIBRARY") or os.path.join(_HERE, "lib", "libmamba_scan.so")

F32, BF16 = 0, 1
STATUS = {
    0: "MAMBA_SCAN_OK", 1: "MAMBA_SCAN_ERR_NULL", 2: "MAMBA_SCAN_ERR_SHAPE", 3: "MAMBA_SCAN_ERR_DTYPE",
    4: "MAMBA_SCAN_ERR_ALIGN", 5: "MAMBA_SCAN_ERR_UNSUPPORTED", 6: "MAMBA_SCAN_ERR_WORKSPACE",
    7: "MAMBA_SCAN_ERR_HIP",
}
EXPORTED = (
    "mamba_scan_fwd", "mamba_scan_fwd_ex", "mamba_scan_fwd_noalloc", "mamba_scan_fwd_workspace_size",
    "mamba_scan_fwd_workspace_size_ex",
    "mamba_scan_fwd_conv",
    "mamba_scan_fwd_varlen", "mamba_scan_fwd_varlen_workspace_size", "mamba_scan_step", "mamba_scan_bwd",
    "mamba_scan_bwd_workspace_size", "mamba_conv1d_fwd", "mamba_ssd_fwd", "mamba_scan_status_str",
    "mamba_scan_abi_version",
)

_lib = None


class MambaScanError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({msg})")
        self.code = code


def load_library():
    """Loads libmamba_scan.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m selective_state_space_55_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.mamba_scan_fwd.restype = I
    lib.mamba_scan_fwd.argtypes = [P] * 11 + [I64] * 4 + [I, I, P, SZ, P]
    lib.mamba_scan_fwd_noalloc.restype = I
    lib.mamba_scan_fwd_noalloc.argtypes = [P] * 11 + [I64] * 4 + [I, I, P]
    lib.mamba_scan_fwd_ex.restype = I
    lib.mamba_scan_fwd_ex.argtypes = [P] * 11 + [I64] * 4 + [I, I, I64, I, P, SZ, P]
    lib.mamba_scan_fwd_workspace_size.restype = SZ
    lib.mamba_scan_fwd_workspace_size.argtypes = [I64] * 4 + [I]
    lib.mamba_scan_fwd_conv.restype = I
    lib.mamba_scan_fwd_conv.argtypes = [P] * 16 + [I64] * 4 + [I, I, P, SZ, P]
    lib.mamba_scan_fwd_workspace_size_ex.restype = SZ
    lib.mamba_scan_fwd_workspace_size_ex.argtypes = [I64] * 4 + [I, I64, I]
    lib.mamba_scan_step.restype = I
    lib.mamba_scan_step.argtypes = [P] * 9 + [I, P] + [I64] * 3 + [I, P]
    lib.mamba_scan_bwd.restype = I
    lib.mamba_scan_bwd.argtypes = [P] * 20 + [I64] * 4 + [I, I, P, SZ, P]
    lib.mamba_scan_bwd_workspace_size.restype = SZ
    lib.mamba_scan_bwd_workspace_size.argtypes = [I64] * 4 + [I]
    lib.mamba_scan_fwd_varlen.restype = I
    lib.mamba_scan_fwd_varlen.argtypes = [P] * 12 + [I64] * 4 + [I, I, P, SZ, P]
    lib.mamba_scan_fwd_varlen_workspace_size.restype = SZ
    lib.mamba_scan_fwd_varlen_workspace_size.argtypes = [I64] * 4 + [I]
    lib.mamba_ssd_fwd.restype = I
    lib.mamba_ssd_fwd.argtypes = [P] * 11 + [I64] * 5 + [I, I, P]
    lib.mamba_conv1d_fwd.restype = I
    lib.mamba_conv1d_fwd.argtypes = [P] * 6 + [I64] * 4 + [I, I, P]
    lib.mamba_scan_status_str.restype = ctypes.c_char_p
    lib.mamba_scan_status_str.argtypes = [I]
    lib.mamba_scan_abi_version.restype = I
    lib.mamba_scan_abi_version.argtypes = []
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().mamba_scan_abi_version())


def status_str(code: int) -> str:
    return load_library().mamba_scan_status_str(int(code)).decode()


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise MambaScanError(fn, code, status_str(code))


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"io tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _req(name: str, t: Optional[torch.Tensor], shape, dtype, device) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


FLAG_SOFTPLUS, FLAG_EULER = 1, 2


def _flags(softplus: bool, discretization: str) -> int:
    if discretization not in ("zoh", "euler"):
        raise ValueError(f"discretization must be 'zoh' or 'euler', got {discretization!r}")
    return (FLAG_SOFTPLUS if softplus else 0) | (FLAG_EULER if discretization == "euler" else 0)


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _on_stream(fn):
    """Runs fn with its `stream` argument made the current stream, so that the outputs and workspace fn
    allocates belong to the stream its kernels are enqueued on (a raw handle is wrapped as an
    ExternalStream of the first argument's device)."""

    @functools.wraps(fn)
    def run(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, stream=None, **kwargs)
        t0 = args[0] if args else None
        dev = t0.device if isinstance(t0, torch.Tensor) else torch.device("cuda", torch.cuda.current_device())
        if not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(int(stream), device=dev)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)

    return run


def fwd_workspace_size(batch: int, dim: int, dstate: int, seqlen: int, io_dtype: int = BF16, nchunks: int = 0,
                       states_per_wave: int = 0) -> int:
    n = load_library().mamba_scan_fwd_workspace_size_ex(batch, dim, dstate, seqlen, io_dtype, nchunks,
                                                        states_per_wave)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("mamba_scan_fwd_workspace_size: sizes rejected")
    return int(n)


@_on_stream
def scan_fwd(u: torch.Tensor, delta: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
             D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
             delta_bias: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
             delta_softplus: bool = True, return_final_state: bool = False, *,
             out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, nchunks: int = 0, states_per_wave: int = 0,
             discretization: str = "zoh", stream=None):
    """Selective-scan forward (discretization "zoh", or "euler" for Bbar u = Delta B u).  u, delta, z: (batch, dim, L); B, C: (batch, dstate, L) in the io dtype
    (float32 or bfloat16); A_log (dim, dstate), D, delta_bias (dim,), initial_state (batch, dim, dstate)
    in float32.  Returns y (batch, dim, L), or (y, final_state) if return_final_state."""
    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, L)")
    batch, dim, L = u.shape
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("scan_fwd needs device tensors (HIP)")
    io = _io_dtype(u)
    iot = u.dtype
    dstate = A_log.shape[-1] if A_log.dim() == 2 else -1
    _req("u", u, (batch, dim, L), iot, dev)
    _req("delta", delta, (batch, dim, L), iot, dev)
    _req("A_log", A_log, (dim, dstate), torch.float32, dev)
    _req("B", B, (batch, dstate, L), iot, dev)
    _req("C", C, (batch, dstate, L), iot, dev)
    _req("D", D, (dim,), torch.float32, dev)
    _req("z", z, (batch, dim, L), iot, dev)
    _req("delta_bias", delta_bias, (dim,), torch.float32, dev)
    _req("initial_state", initial_state, (batch, dim, dstate), torch.float32, dev)
    y = out if out is not None else torch.empty((batch, dim, L), dtype=iot, device=dev)
    _req("out", y, (batch, dim, L), iot, dev)
    fs = final_state
    if fs is None and return_final_state:
        fs = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
    _req("final_state", fs, (batch, dim, dstate), torch.float32, dev)
    need = fwd_workspace_size(batch, dim, dstate, L, io, nchunks, states_per_wave)
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = None, 0
    if ws is not None:
        base = ws.data_ptr()
        off = (-base) % 256
        ws_ptr, ws_bytes = ctypes.c_void_p(base + off), max(0, ws.numel() * ws.element_size() - off)
    rc = lib.mamba_scan_fwd_ex(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(delta_bias), _ptr(initial_state), _ptr(fs), _ptr(y), batch, dim, dstate, L, io,
                               _flags(delta_softplus, discretization), int(nchunks), int(states_per_wave), ws_ptr,
                               ws_bytes,
                               _stream(dev, stream))
    _check("mamba_scan_fwd", rc)
    return (y, fs) if return_final_state else y


NOALLOC_SCRATCH_BYTES = 64 << 20   # MAMBA_SCAN_NOALLOC_SCRATCH_BYTES


@_on_stream
def scan_fwd_noalloc(u: torch.Tensor, delta: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                     out: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                     delta_bias: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                     final_state: Optional[torch.Tensor] = None, delta_softplus: bool = True,
                     discretization: str = "zoh", stream=None) -> torch.Tensor:
    """scan_fwd through mamba_scan_fwd_noalloc: the caller passes every output (out: y, and optionally
    final_state) and nothing is allocated, by this function or the library (the chunk carry lives in
    the library's static per-GPU scratch).  Calls that overlap in time on one GPU race on that scratch.
    Returns out."""
    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, L)")
    batch, dim, L = u.shape
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("scan_fwd_noalloc needs device tensors (HIP)")
    io = _io_dtype(u)
    iot = u.dtype
    dstate = A_log.shape[-1] if A_log.dim() == 2 else -1
    for name, t, shape, dt in (("u", u, (batch, dim, L), iot), ("delta", delta, (batch, dim, L), iot),
                               ("A_log", A_log, (dim, dstate), torch.float32), ("B", B, (batch, dstate, L), iot),
                               ("C", C, (batch, dstate, L), iot), ("D", D, (dim,), torch.float32),
                               ("z", z, (batch, dim, L), iot), ("delta_bias", delta_bias, (dim,), torch.float32),
                               ("initial_state", initial_state, (batch, dim, dstate), torch.float32),
                               ("out", out, (batch, dim, L), iot),
                               ("final_state", final_state, (batch, dim, dstate), torch.float32)):
        _req(name, t, shape, dt, dev)
    if out is None:
        raise ValueError("scan_fwd_noalloc needs out (y)")
    rc = lib.mamba_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                    _ptr(delta_bias), _ptr(initial_state), _ptr(final_state), _ptr(out), batch, dim,
                                    dstate, L, io, _flags(delta_softplus, discretization), _stream(dev, stream))
    _check("mamba_scan_fwd_noalloc", rc)
    return out


@_on_stream
def scan_fwd_conv(x: torch.Tensor, conv_weight: torch.Tensor, delta: torch.Tensor, A_log: torch.Tensor,
                  B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                  delta_bias: Optional[torch.Tensor] = None, conv_bias: Optional[torch.Tensor] = None,
                  conv_state: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                  delta_softplus: bool = True, return_final_state: bool = False, return_conv_state: bool = False,
                  return_u: bool = False, *, out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None, conv_state_out: Optional[torch.Tensor] = None,
                  u_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  discretization: str = "zoh", stream=None):
    """Causal depthwise conv1d (4 taps) + SiLU fused into the forward scan: u = SiLU(conv(x)) is formed
    on chip.  x, delta, z: (batch, dim, L) and B, C: (batch, dstate <= 16, L) in the io dtype;
    conv_weight (dim, 4), conv_bias (dim,), A_log (dim, dstate), D, delta_bias (dim,) float32;
    conv_state (batch, dim, 3) in the io dtype.  Returns y, followed by the final state, the final
    conv state and u for each of return_final_state, return_conv_state, return_u that is set."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, dim, L)")
    batch, dim, L = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("scan_fwd_conv needs device tensors (HIP)")
    io = _io_dtype(x)
    iot = x.dtype
    dstate = A_log.shape[-1] if A_log.dim() == 2 else -1
    _req("x", x, (batch, dim, L), iot, dev)
    _req("conv_weight", conv_weight, (dim, 4), torch.float32, dev)
    _req("conv_bias", conv_bias, (dim,), torch.float32, dev)
    _req("conv_state", conv_state, (batch, dim, 3), iot, dev)
    _req("delta", delta, (batch, dim, L), iot, dev)
    _req("A_log", A_log, (dim, dstate), torch.float32, dev)
    _req("B", B, (batch, dstate, L), iot, dev)
    _req("C", C, (batch, dstate, L), iot, dev)
    _req("D", D, (dim,), torch.float32, dev)
    _req("z", z, (batch, dim, L), iot, dev)
    _req("delta_bias", delta_bias, (dim,), torch.float32, dev)
    _req("initial_state", initial_state, (batch, dim, dstate), torch.float32, dev)
    y = out if out is not None else torch.empty((batch, dim, L), dtype=iot, device=dev)
    _req("out", y, (batch, dim, L), iot, dev)
    fs = final_state
    if fs is None and return_final_state:
        fs = torch.empty((batch, dim, dstate), dtype=torch.float32, device=dev)
    _req("final_state", fs, (batch, dim, dstate), torch.float32, dev)
    cso = conv_state_out
    if cso is None and return_conv_state:
        cso = torch.empty((batch, dim, 3), dtype=iot, device=dev)
    _req("conv_state_out", cso, (batch, dim, 3), iot, dev)
    uo = u_out
    if uo is None and return_u:
        uo = torch.empty((batch, dim, L), dtype=iot, device=dev)
    _req("u_out", uo, (batch, dim, L), iot, dev)
    need = fwd_workspace_size(batch, dim, dstate, L, io)
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = None, 0
    if ws is not None:
        base = ws.data_ptr()
        off = (-base) % 256
        ws_ptr, ws_bytes = ctypes.c_void_p(base + off), max(0, ws.numel() * ws.element_size() - off)
    rc = lib.mamba_scan_fwd_conv(_ptr(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(cso),
                                 _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                 _ptr(initial_state), _ptr(fs), _ptr(uo), _ptr(y), batch, dim, dstate, L, io,
                                 _flags(delta_softplus, discretization), ws_ptr, ws_bytes, _stream(dev, stream))
    _check("mamba_scan_fwd_conv", rc)
    res = [y]
    if return_final_state:
        res.append(fs)
    if return_conv_state:
        res.append(cso)
    if return_u:
        res.append(uo)
    return res[0] if len(res) == 1 else tuple(res)


def fwd_varlen_workspace_size(nseq: int, dim: int, dstate: int, total_len: int, io_dtype: int = BF16) -> int:
    n = load_library().mamba_scan_fwd_varlen_workspace_size(nseq, dim, dstate, total_len, io_dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("mamba_scan_fwd_varlen_workspace_size: sizes rejected")
    return int(n)


@_on_stream
def scan_fwd_varlen(u: torch.Tensor, delta: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                    cu_seqlens: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                    delta_bias: Optional[torch.Tensor] = None, initial_states: Optional[torch.Tensor] = None,
                    delta_softplus: bool = True, return_final_states: bool = False, *,
                    out: Optional[torch.Tensor] = None, final_states: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, discretization: str = "zoh", stream=None):
    """Variable-length batch: nseq sequences packed along time.  u, delta, z: (dim, total); B, C:
    (dstate, total) in the io dtype; cu_seqlens (nseq + 1,) int64 on the device; initial_states
    (nseq, dim, dstate) float32.  Returns y (dim, total), or (y, final_states)."""
    lib = load_library()
    if u.dim() != 2:
        raise ValueError("u must be (dim, total)")
    dim, total = u.shape
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("scan_fwd_varlen needs device tensors (HIP)")
    io = _io_dtype(u)
    iot = u.dtype
    dstate = A_log.shape[-1] if A_log.dim() == 2 else -1
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be (nseq + 1,)")
    nseq = cu_seqlens.numel() - 1
    _req("cu_seqlens", cu_seqlens, (nseq + 1,), torch.int64, dev)
    _req("u", u, (dim, total), iot, dev)
    _req("delta", delta, (dim, total), iot, dev)
    _req("A_log", A_log, (dim, dstate), torch.float32, dev)
    _req("B", B, (dstate, total), iot, dev)
    _req("C", C, (dstate, total), iot, dev)
    _req("D", D, (dim,), torch.float32, dev)
    _req("z", z, (dim, total), iot, dev)
    _req("delta_bias", delta_bias, (dim,), torch.float32, dev)
    _req("initial_states", initial_states, (nseq, dim, dstate), torch.float32, dev)
    y = out if out is not None else torch.empty((dim, total), dtype=iot, device=dev)
    _req("out", y, (dim, total), iot, dev)
    fs = final_states
    if fs is None and return_final_states:
        fs = torch.empty((nseq, dim, dstate), dtype=torch.float32, device=dev)
    _req("final_states", fs, (nseq, dim, dstate), torch.float32, dev)
    need = fwd_varlen_workspace_size(nseq, dim, dstate, total, io)
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = None, 0
    if ws is not None:
        base = ws.data_ptr()
        off = (-base) % 256
        ws_ptr, ws_bytes = ctypes.c_void_p(base + off), max(0, ws.numel() * ws.element_size() - off)
    rc = lib.mamba_scan_fwd_varlen(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                   _ptr(delta_bias), _ptr(cu_seqlens), _ptr(initial_states), _ptr(fs), _ptr(y),
                                   nseq, dim, dstate, total, io, _flags(delta_softplus, discretization), ws_ptr,
                                   ws_bytes, _stream(dev, stream))
    _check("mamba_scan_fwd_varlen", rc)
    return (y, fs) if return_final_states else y


@_on_stream
def scan_step(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor,
              C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
              dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = True, *,
              out: Optional[torch.Tensor] = None, discretization: str = "zoh", stream=None) -> torch.Tensor:
    """One recurrent step (discretization as in scan_fwd).  state (batch, dim, dstate) float32 is updated IN PLACE; x, dt, z (batch, dim)
    and B, C (batch, dstate) in the io dtype.  Returns y (batch, dim)."""
    lib = load_library()
    if state.dim() != 3:
        raise ValueError("state must be (batch, dim, dstate)")
    batch, dim, dstate = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("scan_step needs device tensors (HIP)")
    io = _io_dtype(x)
    iot = x.dtype
    _req("state", state, (batch, dim, dstate), torch.float32, dev)
    _req("x", x, (batch, dim), iot, dev)
    _req("dt", dt, (batch, dim), iot, dev)
    _req("A_log", A_log, (dim, dstate), torch.float32, dev)
    _req("B", B, (batch, dstate), iot, dev)
    _req("C", C, (batch, dstate), iot, dev)
    _req("D", D, (dim,), torch.float32, dev)
    _req("z", z, (batch, dim), iot, dev)
    _req("dt_bias", dt_bias, (dim,), torch.float32, dev)
    y = out if out is not None else torch.empty((batch, dim), dtype=iot, device=dev)
    _req("out", y, (batch, dim), iot, dev)
    rc = lib.mamba_scan_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                             _ptr(dt_bias), _flags(dt_softplus, discretization), _ptr(y), batch, dim, dstate, io,
                             _stream(dev, stream))
    _check("mamba_scan_step", rc)
    return y


def bwd_workspace_size(batch: int, dim: int, dstate: int, seqlen: int, io_dtype: int = BF16) -> int:
    n = load_library().mamba_scan_bwd_workspace_size(batch, dim, dstate, seqlen, io_dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("mamba_scan_bwd_workspace_size: sizes rejected")
    return int(n)


@_on_stream
def scan_bwd(u: torch.Tensor, delta: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
             dy: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
             delta_bias: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
             d_final_state: Optional[torch.Tensor] = None, delta_softplus: bool = True, *,
             workspace: Optional[torch.Tensor] = None, discretization: str = "zoh", stream=None) -> dict:
    """Selective-scan backward.  Inputs as in scan_fwd plus dy (batch, dim, L) in the io dtype and
    d_final_state (batch, dim, dstate) float32.  Returns a dict of gradients: du, ddelta, dz, dB, dC in
    the io dtype; dA_log, dD, ddelta_bias, d_initial_state in float32 (dD, dz, ddelta_bias and
    d_initial_state only when D, z, delta_bias and initial_state are given)."""
    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, L)")
    batch, dim, L = u.shape
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("scan_bwd needs device tensors (HIP)")
    io = _io_dtype(u)
    iot = u.dtype
    dstate = A_log.shape[-1] if A_log.dim() == 2 else -1
    _req("u", u, (batch, dim, L), iot, dev)
    _req("delta", delta, (batch, dim, L), iot, dev)
    _req("A_log", A_log, (dim, dstate), torch.float32, dev)
    _req("B", B, (batch, dstate, L), iot, dev)
    _req("C", C, (batch, dstate, L), iot, dev)
    _req("dy", dy, (batch, dim, L), iot, dev)
    _req("D", D, (dim,), torch.float32, dev)
    _req("z", z, (batch, dim, L), iot, dev)
    _req("delta_bias", delta_bias, (dim,), torch.float32, dev)
    _req("initial_state", initial_state, (batch, dim, dstate), torch.float32, dev)
    _req("d_final_state", d_final_state, (batch, dim, dstate), torch.float32, dev)
    f32 = torch.float32
    g = {"du": torch.empty((batch, dim, L), dtype=iot, device=dev),
         "ddelta": torch.empty((batch, dim, L), dtype=iot, device=dev),
         "dA_log": torch.empty((dim, dstate), dtype=f32, device=dev),
         "dB": torch.empty((batch, dstate, L), dtype=iot, device=dev),
         "dC": torch.empty((batch, dstate, L), dtype=iot, device=dev),
         "dD": torch.empty((dim,), dtype=f32, device=dev) if D is not None else None,
         "dz": torch.empty((batch, dim, L), dtype=iot, device=dev) if z is not None else None,
         "ddelta_bias": torch.empty((dim,), dtype=f32, device=dev) if delta_bias is not None else None,
         "d_initial_state": torch.empty((batch, dim, dstate), dtype=f32, device=dev)
         if initial_state is not None else None}
    need = bwd_workspace_size(batch, dim, dstate, L, io)
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = None, 0
    if ws is not None:
        base = ws.data_ptr()
        off = (-base) % 256
        ws_ptr, ws_bytes = ctypes.c_void_p(base + off), max(0, ws.numel() * ws.element_size() - off)
    rc = lib.mamba_scan_bwd(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                            _ptr(delta_bias), _ptr(initial_state), _ptr(dy), _ptr(d_final_state), _ptr(g["du"]),
                            _ptr(g["ddelta"]), _ptr(g["dA_log"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
                            _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["d_initial_state"]), batch, dim, dstate,
                            L, io, _flags(delta_softplus, discretization), ws_ptr, ws_bytes, _stream(dev, stream))
    _check("mamba_scan_bwd", rc)
    return g


@_on_stream
def conv1d_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
               conv_state: Optional[torch.Tensor] = None, silu: bool = True, return_state: bool = False, *,
               out: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None, stream=None):
    """Causal depthwise conv1d (+ SiLU).  x (batch, dim, L) in the io dtype, weight (dim, K) float32 with
    K <= 4, bias (dim,) float32, conv_state (batch, dim, K-1) in the io dtype (inputs before x, oldest
    first).  Returns u (batch, dim, L), or (u, final conv state) if return_state (state_out may be
    conv_state itself, for an in-place update)."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, dim, L)")
    batch, dim, L = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("conv1d_fwd needs device tensors (HIP)")
    io = _io_dtype(x)
    iot = x.dtype
    K = weight.shape[-1] if weight.dim() == 2 else -1
    _req("weight", weight, (dim, K), torch.float32, dev)
    _req("bias", bias, (dim,), torch.float32, dev)
    _req("conv_state", conv_state, (batch, dim, K - 1), iot, dev)
    u = out if out is not None else torch.empty((batch, dim, L), dtype=iot, device=dev)
    _req("out", u, (batch, dim, L), iot, dev)
    so = state_out
    if so is None and return_state:
        so = torch.empty((batch, dim, K - 1), dtype=iot, device=dev)
    _req("state_out", so, (batch, dim, K - 1), iot, dev)
    rc = lib.mamba_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state), _ptr(so), _ptr(u), batch, dim,
                              L, K, io, int(bool(silu)), _stream(dev, stream))
    _check("mamba_conv1d_fwd", rc)
    return (u, so) if return_state else u


@_on_stream
def ssd_fwd(x: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
            D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
            dt_bias: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
            dt_softplus: bool = True, return_final_state: bool = False, *, out: Optional[torch.Tensor] = None,
            final_state: Optional[torch.Tensor] = None, discretization: str = "zoh", stream=None):
    """Multi-head SSM with a scalar decay per head (state-space-duality form).  x, z: (batch, L, H, P);
    dt: (batch, L, H); B, C: (batch, L, N) in bfloat16; A_log, D, dt_bias: (H,) float32;
    initial_state (batch, H, P, N) float32.  Returns y (batch, L, H, P), or (y, final_state)."""
    lib = load_library()
    if x.dim() != 4:
        raise ValueError("x must be (batch, L, H, P)")
    batch, L, H, P = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_fwd needs device tensors (HIP)")
    io = _io_dtype(x)
    iot = x.dtype
    N = B.shape[-1] if B.dim() == 3 else -1
    _req("x", x, (batch, L, H, P), iot, dev)
    _req("dt", dt, (batch, L, H), iot, dev)
    _req("A_log", A_log, (H,), torch.float32, dev)
    _req("B", B, (batch, L, N), iot, dev)
    _req("C", C, (batch, L, N), iot, dev)
    _req("D", D, (H,), torch.float32, dev)
    _req("z", z, (batch, L, H, P), iot, dev)
    _req("dt_bias", dt_bias, (H,), torch.float32, dev)
    _req("initial_state", initial_state, (batch, H, P, N), torch.float32, dev)
    y = out if out is not None else torch.empty((batch, L, H, P), dtype=iot, device=dev)
    _req("out", y, (batch, L, H, P), iot, dev)
    fs = final_state
    if fs is None and return_final_state:
        fs = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    _req("final_state", fs, (batch, H, P, N), torch.float32, dev)
    rc = lib.mamba_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias),
                           _ptr(initial_state), _ptr(fs), _ptr(y), batch, L, H, P, N, io,
                           _flags(dt_softplus, discretization), _stream(dev, stream))
    _check("mamba_ssd_fwd", rc)
    return (y, fs) if return_final_state else y
