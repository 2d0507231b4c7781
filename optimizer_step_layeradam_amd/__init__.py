"""LayerAdam on MI355X: Python binding of liblayeradam.so.

Argument marshalling only. Every step of the update (gradient sum, unscale,
overflow flag, moments, AdamW step, BF16 cast) runs in the library's HIP
kernel; this module turns torch tensors into the C descriptors of
``include/layeradam.h`` and passes the current HIP stream. PyTorch provides
device memory and streams.

The library must be built (``python -m optimizer_step_layeradam_amd.build``);
there is no fallback: without it every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblayeradam.so")

MAX_REPLICAS = 8
MAX_TENSORS = 256
ALIGNMENT = 16

LA_OK = 0
STATUS_NAMES = {0: "LA_OK", 1: "LA_ERR_INVALID_ARGUMENT", 2: "LA_ERR_MISALIGNED",
                3: "LA_ERR_ALIASING", 4: "LA_ERR_UNSUPPORTED", 5: "LA_ERR_HIP"}
GRAD_BF16, GRAD_FP16 = 0, 1

# Exported symbols, as declared in include/layeradam.h.
EXPORTS = ("layer_adam_step", "la_state_bytes", "la_traffic_bytes", "la_last_error",
           "la_version")


class TensorDesc(ctypes.Structure):
    _fields_ = [("master", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p),
                ("weight_bf16", ctypes.c_void_p),
                ("grads", ctypes.c_void_p * MAX_REPLICAS),
                ("numel", ctypes.c_int64)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("tensors", ctypes.POINTER(TensorDesc)),
                ("num_tensors", ctypes.c_int32),
                ("num_replicas", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32)]


class AdamParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double),
                ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64),
                ("grad_unscale", ctypes.c_double)]


class LayerAdamError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def _single_hip_runtime() -> None:
    """Refuse to run with two HIP runtimes mapped: the library must bind to
    the one torch loaded, or torch's streams and pointers mean nothing to it."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(f"two HIP runtimes are loaded: {sorted(real)}")


def load(path: Optional[str] = None):
    """Load liblayeradam.so once. Import torch first, so that the library
    binds to torch's HIP runtime (both carry the soname libamdhip64.so.7)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m optimizer_step_layeradam_amd.build` "
            "(there is no fallback path)")
    try:
        import torch  # noqa: F401  (loads torch's libamdhip64 first)
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    lib.layer_adam_step.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(AdamParams),
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.layer_adam_step.restype = ctypes.c_int
    lib.la_state_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
    lib.la_state_bytes.restype = ctypes.c_int64
    lib.la_traffic_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
    lib.la_traffic_bytes.restype = ctypes.c_int64
    lib.la_last_error.argtypes = []
    lib.la_last_error.restype = ctypes.c_char_p
    lib.la_version.argtypes = []
    lib.la_version.restype = ctypes.c_char_p
    _single_hip_runtime()
    if path is None:
        _lib = lib
    return lib


def version() -> str:
    return load().la_version().decode()


def last_error() -> str:
    return load().la_last_error().decode()


# ---------------------------------------------------------------------------
# Raw descriptors (plain integers as pointers)
# ---------------------------------------------------------------------------
def make_layer(tensors: Sequence[dict], num_replicas: int, grad_dtype: int):
    """Build a LayerDesc from dicts with integer pointers: master, exp_avg,
    exp_avg_sq, weight_bf16, grads (list of R), numel. Returns (desc, keepalive)."""
    arr = (TensorDesc * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i].master = t.get("master") or 0
        arr[i].exp_avg = t.get("exp_avg") or 0
        arr[i].exp_avg_sq = t.get("exp_avg_sq") or 0
        arr[i].weight_bf16 = t.get("weight_bf16") or 0
        for r, g in enumerate(t.get("grads", ())):
            arr[i].grads[r] = g or 0
        arr[i].numel = int(t["numel"])
    desc = LayerDesc(ctypes.cast(arr, ctypes.POINTER(TensorDesc)), len(tensors),
                     num_replicas, grad_dtype)
    return desc, arr


def make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale=1.0) -> AdamParams:
    return AdamParams(float(lr), float(beta1), float(beta2), float(eps),
                      float(weight_decay), int(step), float(grad_unscale))


def step_raw(desc: LayerDesc, params: AdamParams, overflow_flag: int = 0,
             stream: int = 0) -> None:
    """Call layer_adam_step on raw descriptors; raise LayerAdamError on failure."""
    lib = load()
    rc = lib.layer_adam_step(ctypes.byref(desc), ctypes.byref(params),
                             overflow_flag or None, stream or None)
    if rc != LA_OK:
        raise LayerAdamError(rc, lib.la_last_error().decode())


def state_bytes_raw(desc: LayerDesc) -> int:
    return load().la_state_bytes(ctypes.byref(desc))


def traffic_bytes_raw(desc: LayerDesc) -> int:
    return load().la_traffic_bytes(ctypes.byref(desc))


# ---------------------------------------------------------------------------
# torch tensors
# ---------------------------------------------------------------------------
def _grad_dtype_of(grads) -> int:
    import torch
    kinds = {g.dtype for gs in grads for g in gs}
    if kinds <= {torch.bfloat16}:
        return GRAD_BF16
    if kinds <= {torch.float16}:
        return GRAD_FP16
    raise TypeError(f"gradients must all be bfloat16 or all float16, got {kinds}")


def _describe(params, grads):
    import torch
    if len(params) != len(grads):
        raise ValueError("one list of gradient replicas per tensor")
    if not params:
        return [], 1, GRAD_BF16
    R = len(grads[0])
    gd = _grad_dtype_of(grads)
    out = []
    for i, ((p, m, v, w), gs) in enumerate(zip(params, grads)):
        n = p.numel()
        for name, x, dt in (("master", p, torch.float32), ("exp_avg", m, torch.float32),
                            ("exp_avg_sq", v, torch.float32),
                            ("weight_bf16", w, torch.bfloat16)):
            if x.dtype != dt and not (name == "weight_bf16" and x.dtype in (torch.int16,)):
                raise TypeError(f"tensor {i}: {name} must be {dt}, got {x.dtype}")
            if x.numel() != n or not x.is_contiguous() or not x.is_cuda:
                raise ValueError(f"tensor {i}: {name} must be a contiguous CUDA tensor "
                                 f"of {n} elements")
        if len(gs) != R:
            raise ValueError(f"tensor {i}: {len(gs)} gradient replicas, expected {R}")
        for g in gs:
            if g.numel() != n or not g.is_contiguous() or not g.is_cuda:
                raise ValueError(f"tensor {i}: gradients must be contiguous CUDA tensors "
                                 f"of {n} elements")
        out.append(dict(master=p.data_ptr(), exp_avg=m.data_ptr(), exp_avg_sq=v.data_ptr(),
                        weight_bf16=w.data_ptr(), grads=[g.data_ptr() for g in gs], numel=n))
    return out, R, gd


def step(params, grads, *, lr: float, beta1: float, beta2: float, eps: float,
         weight_decay: float, step: int, grad_unscale: float = 1.0,
         overflow_flag=None, stream=None) -> None:
    """One LayerAdam update of a layer, enqueued on ``stream`` (default: the
    current torch stream).

    params: per tensor a tuple (master fp32, exp_avg fp32, exp_avg_sq fp32,
            weight_bf16 bf16), updated/written in place.
    grads:  per tensor a list of R gradient replicas (all bf16 or all fp16).
    overflow_flag: optional int32 CUDA tensor of one element (set to 1 on a
            non-finite aggregated gradient; never cleared).
    """
    import torch
    tensors, R, gd = _describe(params, grads)
    desc, keep = make_layer(tensors, R, gd)
    hp = make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale)
    flag_ptr = 0
    if overflow_flag is not None:
        if overflow_flag.dtype != torch.int32 or not overflow_flag.is_cuda:
            raise TypeError("overflow_flag must be an int32 CUDA tensor")
        flag_ptr = overflow_flag.data_ptr()
    s = stream if stream is not None else torch.cuda.current_stream()
    step_raw(desc, hp, flag_ptr, s.cuda_stream)
    del keep


def state_bytes(numels: Sequence[int], num_replicas: int = 1) -> int:
    """16 bytes per parameter (la_state_bytes)."""
    desc, keep = make_layer([dict(numel=n) for n in numels], num_replicas, GRAD_BF16)
    return state_bytes_raw(desc)


def traffic_bytes(numels: Sequence[int], num_replicas: int) -> int:
    """(2R + 26) bytes per parameter (la_traffic_bytes)."""
    desc, keep = make_layer([dict(numel=n) for n in numels], num_replicas, GRAD_BF16)
    return traffic_bytes_raw(desc)
