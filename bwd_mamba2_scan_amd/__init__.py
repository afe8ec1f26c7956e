"""Python binding of libmamba2scan.so, the MI355X Mamba2 temporal scan.

Argument marshalling only: every step of the forward and backward runs in the
library's HIP kernels.  PyTorch supplies device memory and the stream.  There
is no CPU or PyTorch fallback: if the library is not built, every call raises.

The entry points mirror include/mamba2_scan.h:
    fwd(h_history, h_s2, W_A, W_B, W_C)         -> (context, saved)
        (h_history and h_s2 float32, or both bfloat16 for the *_bf16 entry points)
    bwd(h_history, h_s2, saved, d_context)      -> dict(dW_A, dW_B, dW_C[, d_a, d_b, d_c])
    bwd_partials(...), bwd_reduce(...)          -- the two phases of bwd
    bwd_input(W_A, W_B, W_C, saved, d_context, K) -> (d_h_history, d_h_s2)
    bwd_full(h_history, h_s2, saved, d_context, W_A, W_B, W_C) -> dict(dW_*, d_h_history, d_h_s2)
    fwd_blend(...) -> (context, h_enriched, saved);  bwd_blend(...) -> dict(...)
    saved_bytes(B, K, SH2, D), workspace_bytes(B, K, SH2, D)
"""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmamba2scan.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "mamba2_scan.h")

OK = 0
EBADDIM = -1
EUNSUPPORTED = -2
ENULL = -3
ESIZE = -4
EALIGN = -5
EHIP = -6
ESCRATCH = -7


class Mamba2ScanError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib = None

_c_int = ctypes.c_int
_c_size = ctypes.c_size_t
_c_vp = ctypes.c_void_p

_SIGNATURES = {
    "mamba2_scan_saved_bytes": (_c_size, [_c_int] * 4),
    "mamba2_scan_bwd_workspace_bytes": (_c_size, [_c_int] * 4),
    "mamba2_scan_fwd": (_c_int, [_c_int] * 4 + [_c_vp] * 7 + [_c_size, _c_vp]),
    "mamba2_scan_bwd": (_c_int, [_c_int] * 4 + [_c_vp] * 3 + [_c_size] + [_c_vp] * 8 + [_c_size, _c_vp]),
    "mamba2_scan_bwd_partials": (_c_int, [_c_int] * 4 + [_c_vp] * 3 + [_c_size] + [_c_vp] * 5 + [_c_size, _c_vp]),
    "mamba2_scan_bwd_reduce": (_c_int, [_c_int] * 4 + [_c_vp, _c_size] + [_c_vp] * 4),
    "mamba2_scan_bwd_input": (_c_int, [_c_int] * 4 + [_c_vp] * 4 + [_c_size] + [_c_vp] * 4),
    "mamba2_scan_fwd_blend": (_c_int, [_c_int] * 4 + [_c_vp] * 10 + [_c_size, _c_vp]),
    "mamba2_scan_bwd_blend_workspace_bytes": (_c_size, [_c_int] * 4),
    "mamba2_scan_bwd_blend": (_c_int, [_c_int] * 4 + [_c_vp] * 3 + [_c_size] + [_c_vp] * 8 + [_c_size, _c_vp]),
    "mamba2_scan_fwd_bf16": (_c_int, [_c_int] * 4 + [_c_vp] * 7 + [_c_size, _c_vp]),
    "mamba2_scan_bwd_bf16": (_c_int, [_c_int] * 4 + [_c_vp] * 3 + [_c_size] + [_c_vp] * 8 + [_c_size, _c_vp]),
    "mamba2_scan_bwd_partials_bf16": (_c_int, [_c_int] * 4 + [_c_vp] * 3 + [_c_size] + [_c_vp] * 5 + [_c_size, _c_vp]),
    "mamba2_scan_strerror": (ctypes.c_char_p, [_c_int]),
    "mamba2_scan_fwd_plan": (_c_int, [_c_int] * 4 + [_c_vp, _c_int]),
    "mamba2_scan_bwd_noalloc": (_c_int, [_c_int] * 4 + [_c_vp] * 3 + [_c_size] + [_c_vp] * 8),
    "mamba2_scan_bwd_full": (_c_int, [_c_int] * 4 + [_c_vp] * 3 + [_c_size] + [_c_vp] * 10 + [_c_size, _c_vp]),
    "mamba2_scan_bwd_full_bf16": (_c_int, [_c_int] * 4 + [_c_vp] * 3 + [_c_size] + [_c_vp] * 10 + [_c_size, _c_vp]),
}


class Launch(ctypes.Structure):
    """mamba2_scan_launch: one kernel launch of a forward call."""
    _fields_ = [(n, ctypes.c_int) for n in
                ("kernel", "sample_blocks", "pass_", "chunks", "chunk_steps", "grid", "threads")]


KERNEL_NAMES = {0: "fwd", 1: "carry"}
PASS_NAMES = {0: "full", 1: "summary", 2: "carry", 3: "replay"}


def lib():
    """The loaded ctypes handle; raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bwd_mamba2_scan_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/mamba2_scan.h declares."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba2_scan_\w+)\s*\(", text)))


def strerror(status: int) -> str:
    return lib().mamba2_scan_strerror(status).decode()


def saved_bytes(B: int, K: int, SH2: int, D: int) -> int:
    return int(lib().mamba2_scan_saved_bytes(B, K, SH2, D))


def workspace_bytes(B: int, K: int, SH2: int, D: int) -> int:
    return int(lib().mamba2_scan_bwd_workspace_bytes(B, K, SH2, D))


def fwd_plan(B: int, K: int, SH2: int, D: int) -> list[dict]:
    """The kernel launches a forward call enqueues for these dimensions (host only, no GPU)."""
    buf = (Launch * 4)()
    n = lib().mamba2_scan_fwd_plan(B, K, SH2, D, ctypes.cast(buf, ctypes.c_void_p), 4)
    _raise(n if n < 0 else OK, "mamba2_scan_fwd_plan")
    return [{"kernel": KERNEL_NAMES[l.kernel], "sample_blocks": l.sample_blocks, "pass": PASS_NAMES[l.pass_],
             "chunks": l.chunks, "chunk_steps": l.chunk_steps, "grid": l.grid, "threads": l.threads}
            for l in buf[:n]]


# ----------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, device, dtype=None):
    torch = _torch()
    dtype = torch.float32 if dtype is None else dtype
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dims(h_history, D):
    B, K, SH2 = (int(v) for v in h_history.shape)
    return B, K, SH2, int(D)


def _trunk_dtype(h_history):
    """float32, or bfloat16 for the reduced-precision trunk entry points."""
    torch = _torch()
    if h_history.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"h_history must be float32 or bfloat16 (got {h_history.dtype})")
    return h_history.dtype


def _is_bf16(dtype):
    return dtype == _torch().bfloat16


def _raise(status, where):
    if status != OK:
        raise Mamba2ScanError(status, where)


def alloc_saved(B, K, SH2, D, device):
    torch = _torch()
    n = saved_bytes(B, K, SH2, D)
    if n == 0:
        raise ValueError(f"unsupported dimensions B={B} K={K} SH2={SH2} D={D}")
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def alloc_workspace(B, K, SH2, D, device):
    torch = _torch()
    n = workspace_bytes(B, K, SH2, D)
    if n == 0:
        raise ValueError(f"unsupported dimensions B={B} K={K} SH2={SH2} D={D}")
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def fwd(h_history, h_s2, W_A, W_B, W_C, *, context=None, saved=None, stream=None):
    """Forward scan.  Returns (context [B, D], saved) -- saved feeds bwd()."""
    torch = _torch()
    if h_history.dim() != 3 or W_A.dim() != 2:
        raise ValueError("h_history must be [B, K, SH2] and W_A [SH2, D]")
    B, K, SH2, D = _dims(h_history, W_A.shape[1])
    dev = h_history.device
    tdt = _trunk_dtype(h_history)
    _check(h_history, "h_history", (B, K, SH2), None, tdt)
    _check(h_s2, "h_s2", (B, SH2), dev, tdt)
    for name, w in (("W_A", W_A), ("W_B", W_B), ("W_C", W_C)):
        _check(w, name, (SH2, D), dev)
    if context is None:
        context = torch.empty((B, D), dtype=torch.float32, device=dev)
    _check(context, "context", (B, D), dev)
    if saved is None:
        saved = alloc_saved(B, K, SH2, D, dev)
    _check(saved, "saved", None, dev)
    fn, name = ((lib().mamba2_scan_fwd_bf16, "mamba2_scan_fwd_bf16") if _is_bf16(tdt)
                else (lib().mamba2_scan_fwd, "mamba2_scan_fwd"))
    st = fn(B, K, SH2, D, _ptr(h_history), _ptr(h_s2), _ptr(W_A), _ptr(W_B), _ptr(W_C),
            _ptr(context), _ptr(saved), saved.numel() * 4, _stream(stream, dev))
    _raise(st, name)
    return context, saved


def _bwd_args(h_history, h_s2, saved, d_context):
    if h_history.dim() != 3 or d_context.dim() != 2:
        raise ValueError("h_history must be [B, K, SH2] and d_context [B, D]")
    B, K, SH2, D = _dims(h_history, d_context.shape[1])
    dev = h_history.device
    tdt = _trunk_dtype(h_history)
    _check(h_history, "h_history", (B, K, SH2), None, tdt)
    _check(h_s2, "h_s2", (B, SH2), dev, tdt)
    _check(saved, "saved", None, dev)
    _check(d_context, "d_context", (B, D), dev)
    return B, K, SH2, D, dev


def _debug_bufs(debug, B, K, D, dev):
    torch = _torch()
    if not debug:
        return None, None, None
    return (torch.empty((B, K, D), dtype=torch.float32, device=dev),
            torch.empty((B, K, D), dtype=torch.float32, device=dev),
            torch.empty((B, D), dtype=torch.float32, device=dev))


def bwd(h_history, h_s2, saved, d_context, *, workspace=None, out=None, debug=False, stream=None):
    """Backward scan.  Returns dict with dW_A, dW_B, dW_C [SH2, D] (and d_a, d_b, d_c if debug)."""
    torch = _torch()
    B, K, SH2, D, dev = _bwd_args(h_history, h_s2, saved, d_context)
    if workspace is None:
        workspace = alloc_workspace(B, K, SH2, D, dev)
    _check(workspace, "workspace", None, dev)
    if out is None:
        out = {n: torch.empty((SH2, D), dtype=torch.float32, device=dev) for n in ("dW_A", "dW_B", "dW_C")}
    for n in ("dW_A", "dW_B", "dW_C"):
        _check(out[n], n, (SH2, D), dev)
    d_a, d_b, d_c = _debug_bufs(debug, B, K, D, dev)
    fn, name = ((lib().mamba2_scan_bwd_bf16, "mamba2_scan_bwd_bf16") if _is_bf16(h_history.dtype)
                else (lib().mamba2_scan_bwd, "mamba2_scan_bwd"))
    st = fn(B, K, SH2, D, _ptr(h_history), _ptr(h_s2), _ptr(saved), saved.numel() * 4,
            _ptr(d_context), _ptr(out["dW_A"]), _ptr(out["dW_B"]), _ptr(out["dW_C"]),
            _ptr(d_a), _ptr(d_b), _ptr(d_c), _ptr(workspace), workspace.numel() * 4,
            _stream(stream, dev))
    _raise(st, name)
    res = dict(out)
    if debug:
        res.update(d_a=d_a, d_b=d_b, d_c=d_c)
    return res


def bwd_full(h_history, h_s2, saved, d_context, W_A, W_B, W_C, *, workspace=None, out=None,
             want=("h_history", "h_s2"), stream=None):
    """Backward with the input gradients (mamba2_scan_bwd_full).

    Returns dict with dW_A, dW_B, dW_C [SH2, D], d_h_history [B, K, SH2] and
    d_h_s2 [B, SH2]; an input gradient not named in `want` (and not passed in
    `out`) comes back as None.
    """
    torch = _torch()
    B, K, SH2, D, dev = _bwd_args(h_history, h_s2, saved, d_context)
    for name, w in (("W_A", W_A), ("W_B", W_B), ("W_C", W_C)):
        _check(w, name, (SH2, D), dev)
    if workspace is None:
        workspace = alloc_workspace(B, K, SH2, D, dev)
    _check(workspace, "workspace", None, dev)
    res = dict(out or {})
    for n in ("dW_A", "dW_B", "dW_C"):
        if res.get(n) is None:
            res[n] = torch.empty((SH2, D), dtype=torch.float32, device=dev)
        _check(res[n], n, (SH2, D), dev)
    shapes = {"d_h_history": (B, K, SH2), "d_h_s2": (B, SH2)}
    for n, shape in shapes.items():
        if res.get(n) is None and n[2:] in want:
            res[n] = torch.empty(shape, dtype=torch.float32, device=dev)
        if res.get(n) is not None:
            _check(res[n], n, shape, dev)
        else:
            res[n] = None
    fn, name = ((lib().mamba2_scan_bwd_full_bf16, "mamba2_scan_bwd_full_bf16") if _is_bf16(h_history.dtype)
                else (lib().mamba2_scan_bwd_full, "mamba2_scan_bwd_full"))
    st = fn(B, K, SH2, D, _ptr(h_history), _ptr(h_s2), _ptr(saved), saved.numel() * 4, _ptr(d_context),
            _ptr(W_A), _ptr(W_B), _ptr(W_C), _ptr(res["dW_A"]), _ptr(res["dW_B"]), _ptr(res["dW_C"]),
            _ptr(res["d_h_history"]), _ptr(res["d_h_s2"]), _ptr(workspace), workspace.numel() * 4,
            _stream(stream, dev))
    _raise(st, name)
    return res


def bwd_partials(h_history, h_s2, saved, d_context, workspace, *, debug=False, stream=None):
    """Phase 1 of bwd: writes the split-K partial slices into `workspace`."""
    B, K, SH2, D, dev = _bwd_args(h_history, h_s2, saved, d_context)
    _check(workspace, "workspace", None, dev)
    d_a, d_b, d_c = _debug_bufs(debug, B, K, D, dev)
    fn, name = ((lib().mamba2_scan_bwd_partials_bf16, "mamba2_scan_bwd_partials_bf16") if _is_bf16(h_history.dtype)
                else (lib().mamba2_scan_bwd_partials, "mamba2_scan_bwd_partials"))
    st = fn(B, K, SH2, D, _ptr(h_history), _ptr(h_s2), _ptr(saved), saved.numel() * 4, _ptr(d_context),
            _ptr(d_a), _ptr(d_b), _ptr(d_c), _ptr(workspace), workspace.numel() * 4, _stream(stream, dev))
    _raise(st, name)
    return dict(d_a=d_a, d_b=d_b, d_c=d_c) if debug else {}


def bwd_reduce(B, K, SH2, D, workspace, dW_A, dW_B, dW_C, *, stream=None):
    """Phase 2 of bwd: fixed-order sum of the slices into dW_A, dW_B, dW_C."""
    dev = workspace.device
    _check(workspace, "workspace", None, dev)
    for name, t in (("dW_A", dW_A), ("dW_B", dW_B), ("dW_C", dW_C)):
        _check(t, name, (SH2, D), dev)
    st = lib().mamba2_scan_bwd_reduce(B, K, SH2, D, _ptr(workspace), workspace.numel() * 4, _ptr(dW_A),
                                      _ptr(dW_B), _ptr(dW_C), _stream(stream, dev))
    _raise(st, "mamba2_scan_bwd_reduce")


def bwd_input(W_A, W_B, W_C, saved, d_context, K, *, d_h_history=None, d_h_s2=None, want=("h_history", "h_s2"),
              stream=None):
    """Input gradients (d_h_history [B, K, SH2], d_h_s2 [B, SH2]) from the forward's saved terms.

    `want` names the outputs to compute; an output not wanted comes back as None.
    """
    torch = _torch()
    if W_A.dim() != 2 or d_context.dim() != 2:
        raise ValueError("W_A must be [SH2, D] and d_context [B, D]")
    SH2, D = (int(v) for v in W_A.shape)
    B = int(d_context.shape[0])
    K = int(K)
    dev = W_A.device
    for name, w in (("W_A", W_A), ("W_B", W_B), ("W_C", W_C)):
        _check(w, name, (SH2, D), dev)
    _check(saved, "saved", None, dev)
    _check(d_context, "d_context", (B, D), dev)
    if "h_history" in want and d_h_history is None:
        d_h_history = torch.empty((B, K, SH2), dtype=torch.float32, device=dev)
    if "h_s2" in want and d_h_s2 is None:
        d_h_s2 = torch.empty((B, SH2), dtype=torch.float32, device=dev)
    if d_h_history is not None:
        _check(d_h_history, "d_h_history", (B, K, SH2), dev)
    if d_h_s2 is not None:
        _check(d_h_s2, "d_h_s2", (B, SH2), dev)
    st = lib().mamba2_scan_bwd_input(B, K, SH2, D, _ptr(W_A), _ptr(W_B), _ptr(W_C), _ptr(saved), saved.numel() * 4,
                                     _ptr(d_context), _ptr(d_h_history), _ptr(d_h_s2), _stream(stream, dev))
    _raise(st, "mamba2_scan_bwd_input")
    return d_h_history, d_h_s2


def blend_workspace_bytes(B: int, K: int, SH2: int, D: int) -> int:
    return int(lib().mamba2_scan_bwd_blend_workspace_bytes(B, K, SH2, D))


def fwd_blend(h_history, h_s2, W_A, W_B, W_C, *, stability=None, temporal_weight=None, context=None,
              h_enriched=None, saved=None, want_h_enriched=True, stream=None):
    """Forward with the stability multiplier and the h_enriched blend.

    stability: a one-element device tensor (m), or None for 1.
    Returns (context, h_enriched or None, saved).
    """
    torch = _torch()
    if h_history.dim() != 3 or W_A.dim() != 2:
        raise ValueError("h_history must be [B, K, SH2] and W_A [SH2, D]")
    B, K, SH2, D = _dims(h_history, W_A.shape[1])
    dev = h_history.device
    _check(h_history, "h_history", (B, K, SH2), None)
    _check(h_s2, "h_s2", (B, SH2), dev)
    for name, w in (("W_A", W_A), ("W_B", W_B), ("W_C", W_C)):
        _check(w, name, (SH2, D), dev)
    if stability is not None:
        _check(stability, "stability", None, dev)
        if stability.numel() < 1:
            raise ValueError("stability must hold one value")
    if temporal_weight is not None:
        _check(temporal_weight, "temporal_weight", (SH2,), dev)
    if context is None:
        context = torch.empty((B, D), dtype=torch.float32, device=dev)
    _check(context, "context", (B, D), dev)
    if h_enriched is None and want_h_enriched:
        h_enriched = torch.empty((B, SH2), dtype=torch.float32, device=dev)
    if h_enriched is not None:
        _check(h_enriched, "h_enriched", (B, SH2), dev)
    if saved is None:
        saved = alloc_saved(B, K, SH2, D, dev)
    _check(saved, "saved", None, dev)
    st = lib().mamba2_scan_fwd_blend(B, K, SH2, D, _ptr(h_history), _ptr(h_s2), _ptr(W_A), _ptr(W_B), _ptr(W_C),
                                     _ptr(stability), _ptr(temporal_weight), _ptr(context), _ptr(h_enriched),
                                     _ptr(saved), saved.numel() * 4, _stream(stream, dev))
    _raise(st, "mamba2_scan_fwd_blend")
    return context, h_enriched, saved


def bwd_blend(h_history, h_s2, saved, d_h_enriched, D, *, temporal_weight=None, want_d_temporal_weight=True,
              workspace=None, out=None, stream=None):
    """Backward of the blend and the scan: dict with dW_A, dW_B, dW_C, d_context, d_temporal_weight.

    D is STATE_D (the blend's inputs do not imply it).
    """
    torch = _torch()
    if h_history.dim() != 3 or d_h_enriched.dim() != 2:
        raise ValueError("h_history must be [B, K, SH2] and d_h_enriched [B, SH2]")
    B, K, SH2 = (int(v) for v in h_history.shape)
    dev = h_history.device
    _check(h_history, "h_history", (B, K, SH2), None)
    _check(h_s2, "h_s2", (B, SH2), dev)
    _check(saved, "saved", None, dev)
    _check(d_h_enriched, "d_h_enriched", (B, SH2), dev)
    if temporal_weight is not None:
        _check(temporal_weight, "temporal_weight", (SH2,), dev)
    D = int(D)
    if out is None:
        out = {n: torch.empty((SH2, D), dtype=torch.float32, device=dev) for n in ("dW_A", "dW_B", "dW_C")}
    for n in ("dW_A", "dW_B", "dW_C"):
        _check(out[n], n, (SH2, D), dev)
    res = dict(out)
    if res.get("d_context") is None:
        res["d_context"] = torch.empty((B, D), dtype=torch.float32, device=dev)
    _check(res["d_context"], "d_context", (B, D), dev)
    if want_d_temporal_weight and res.get("d_temporal_weight") is None:
        res["d_temporal_weight"] = torch.empty((SH2,), dtype=torch.float32, device=dev)
    if res.get("d_temporal_weight") is not None:
        _check(res["d_temporal_weight"], "d_temporal_weight", (SH2,), dev)
    if workspace is None:
        n = blend_workspace_bytes(B, K, SH2, D)
        if n == 0:
            raise ValueError(f"unsupported dimensions B={B} K={K} SH2={SH2} D={D}")
        workspace = torch.empty(n // 4, dtype=torch.float32, device=dev)
    _check(workspace, "workspace", None, dev)
    st = lib().mamba2_scan_bwd_blend(B, K, SH2, D, _ptr(h_history), _ptr(h_s2), _ptr(saved), saved.numel() * 4,
                                     _ptr(temporal_weight), _ptr(d_h_enriched), _ptr(res["d_context"]),
                                     _ptr(res["dW_A"]), _ptr(res["dW_B"]), _ptr(res["dW_C"]),
                                     _ptr(res.get("d_temporal_weight")), _ptr(workspace), workspace.numel() * 4,
                                     _stream(stream, dev))
    _raise(st, "mamba2_scan_bwd_blend")
    return res
