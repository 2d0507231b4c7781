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
OUT_BF16, OUT_FP16, OUT_NONE = 0, 1, 2
PROBE_READS, PROBE_WRITES = 0, 1

# Exported symbols, as declared in include/layeradam.h.
EXPORTS = ("layer_adam_step", "layer_adam_step_range", "layer_adam_step_gated",
           "layer_adam_step_device_step", "layer_adam_step_ex", "la_check_gradients",
           "la_stream_probe",
           "la_direction_probe", "la_copy_reference",
           "la_state_bytes", "la_traffic_bytes", "la_last_error", "la_version")


class TensorDesc(ctypes.Structure):
    _fields_ = [("master", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p),
                ("weight_out", ctypes.c_void_p),
                ("grads", ctypes.c_void_p * MAX_REPLICAS),
                ("numel", ctypes.c_int64)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("tensors", ctypes.POINTER(TensorDesc)),
                ("num_tensors", ctypes.c_int32),
                ("num_replicas", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class AdamParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double),
                ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64),
                ("grad_unscale", ctypes.c_double)]


class StepOptions(ctypes.Structure):
    _fields_ = [("use_range", ctypes.c_int32),
                ("elem_begin", ctypes.c_int64),
                ("elem_end", ctypes.c_int64),
                ("overflow_flag", ctypes.c_void_p),
                ("skip_if_nonzero", ctypes.c_void_p),
                ("step_on_device", ctypes.c_void_p)]


class LayerAdamError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_hip = None


class _PointerAttributes(ctypes.Structure):  # hipPointerAttribute_t
    _fields_ = [("type", ctypes.c_int),
                ("device", ctypes.c_int),
                ("devicePointer", ctypes.c_void_p),
                ("hostPointer", ctypes.c_void_p),
                ("isManaged", ctypes.c_int),
                ("allocationFlags", ctypes.c_uint)]


_HIP_MEMORY_HOST, _HIP_MEMORY_DEVICE = 1, 2


def _hip_runtime():
    """The HIP runtime already mapped into the process (torch's)."""
    global _hip
    if _hip is None:
        with open("/proc/self/maps") as f:
            paths = [line.split()[-1] for line in f if "libamdhip64" in line]
        if not paths:
            raise RuntimeError("no HIP runtime loaded")
        _hip = ctypes.CDLL(paths[0])
        _hip.hipPointerGetAttributes.argtypes = [ctypes.POINTER(_PointerAttributes),
                                                 ctypes.c_void_p]
        _hip.hipPointerGetAttributes.restype = ctypes.c_int
    return _hip


def device_address(t) -> int:
    """Address the kernel may use for tensor t: its data pointer for a CUDA
    tensor; for a pinned (page-locked) host tensor, the device-side address of
    the mapping HIP made when it was allocated. Anything else is refused."""
    if t.is_cuda:
        import torch
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"tensor on {t.device}, but the current device is "
                             f"cuda:{torch.cuda.current_device()}")
        return t.data_ptr()
    if not t.is_pinned():
        raise TypeError("host tensors must be pinned (page-locked, e.g. pin_memory=True)")
    ptr = t.data_ptr()
    attr = _PointerAttributes()
    rc = _hip_runtime().hipPointerGetAttributes(ctypes.byref(attr), ctypes.c_void_p(ptr))
    if rc != 0 or attr.type != _HIP_MEMORY_HOST or not attr.devicePointer:
        raise TypeError(f"pinned host memory at {ptr:#x} is not mapped for the GPU "
                        f"(hipPointerGetAttributes rc={rc}, type={attr.type})")
    return attr.devicePointer + (ptr - (attr.hostPointer or ptr))


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
    lib.layer_adam_step_range.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(AdamParams),
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.layer_adam_step_range.restype = ctypes.c_int
    lib.layer_adam_step_gated.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(AdamParams),
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.layer_adam_step_gated.restype = ctypes.c_int
    lib.layer_adam_step_device_step.argtypes = [ctypes.POINTER(LayerDesc),
                                                ctypes.POINTER(AdamParams), ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p]
    lib.layer_adam_step_device_step.restype = ctypes.c_int
    lib.layer_adam_step_ex.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(AdamParams),
                                       ctypes.POINTER(StepOptions), ctypes.c_void_p]
    lib.layer_adam_step_ex.restype = ctypes.c_int
    lib.la_check_gradients.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_double,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.la_check_gradients.restype = ctypes.c_int
    lib.la_stream_probe.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_void_p]
    lib.la_stream_probe.restype = ctypes.c_int
    lib.la_direction_probe.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32,
                                       ctypes.c_void_p]
    lib.la_direction_probe.restype = ctypes.c_int
    lib.la_copy_reference.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
    lib.la_copy_reference.restype = ctypes.c_int
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
def make_layer(tensors: Sequence[dict], num_replicas: int, grad_dtype: int,
               out_dtype: int = OUT_BF16):
    """Build a LayerDesc from dicts with integer pointers: master, exp_avg,
    exp_avg_sq, weight_out, grads (list of R), numel. Returns (desc, keepalive)."""
    arr = (TensorDesc * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i].master = t.get("master") or 0
        arr[i].exp_avg = t.get("exp_avg") or 0
        arr[i].exp_avg_sq = t.get("exp_avg_sq") or 0
        arr[i].weight_out = t.get("weight_out") or 0
        for r, g in enumerate(t.get("grads", ())):
            arr[i].grads[r] = g or 0
        arr[i].numel = int(t["numel"])
    desc = LayerDesc(ctypes.cast(arr, ctypes.POINTER(TensorDesc)), len(tensors),
                     num_replicas, grad_dtype, out_dtype)
    return desc, arr


def make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale=1.0) -> AdamParams:
    return AdamParams(float(lr), float(beta1), float(beta2), float(eps),
                      float(weight_decay), int(step), float(grad_unscale))


def _raise_on(rc: int, lib) -> None:
    if rc != LA_OK:
        raise LayerAdamError(rc, lib.la_last_error().decode())


def step_raw(desc: LayerDesc, params: AdamParams, overflow_flag: int = 0,
             stream: int = 0) -> None:
    """layer_adam_step on raw descriptors; raises LayerAdamError on failure."""
    lib = load()
    _raise_on(lib.layer_adam_step(ctypes.byref(desc), ctypes.byref(params),
                                  overflow_flag or None, stream or None), lib)


def step_range_raw(desc: LayerDesc, params: AdamParams, begin: int, end: int,
                   overflow_flag: int = 0, stream: int = 0) -> None:
    """layer_adam_step_range on raw descriptors."""
    lib = load()
    _raise_on(lib.layer_adam_step_range(ctypes.byref(desc), ctypes.byref(params), int(begin),
                                        int(end), overflow_flag or None, stream or None), lib)


def step_gated_raw(desc: LayerDesc, params: AdamParams, skip_if_nonzero: int,
                   overflow_flag: int = 0, stream: int = 0) -> None:
    """layer_adam_step_gated on raw descriptors."""
    lib = load()
    _raise_on(lib.layer_adam_step_gated(ctypes.byref(desc), ctypes.byref(params),
                                        skip_if_nonzero or None, overflow_flag or None,
                                        stream or None), lib)


def step_device_step_raw(desc: LayerDesc, params: AdamParams, step_on_device: int,
                         overflow_flag: int = 0, stream: int = 0) -> None:
    """layer_adam_step_device_step on raw descriptors (params.step ignored)."""
    lib = load()
    _raise_on(lib.layer_adam_step_device_step(ctypes.byref(desc), ctypes.byref(params),
                                              step_on_device or None, overflow_flag or None,
                                              stream or None), lib)


def step_ex_raw(desc: LayerDesc, params: AdamParams, begin: Optional[int] = None,
                end: Optional[int] = None, overflow_flag: int = 0, skip_if_nonzero: int = 0,
                step_on_device: int = 0, stream: int = 0) -> None:
    """layer_adam_step_ex on raw descriptors: the element range [begin, end)
    when both are given, else the whole layer; zero pointers mean no flag, no
    skip flag and t from params.step."""
    if (begin is None) != (end is None):
        raise ValueError("give both begin and end, or neither")
    opts = StepOptions(0 if begin is None else 1, int(begin or 0), int(end or 0),
                       overflow_flag or None, skip_if_nonzero or None, step_on_device or None)
    lib = load()
    _raise_on(lib.layer_adam_step_ex(ctypes.byref(desc), ctypes.byref(params),
                                     ctypes.byref(opts), stream or None), lib)


def check_gradients_raw(desc: LayerDesc, grad_unscale: float, found_nonfinite: int,
                        stream: int = 0) -> None:
    """la_check_gradients on raw descriptors."""
    lib = load()
    _raise_on(lib.la_check_gradients(ctypes.byref(desc), float(grad_unscale),
                                     found_nonfinite or None, stream or None), lib)


def stream_probe_raw(desc: LayerDesc, stream: int = 0) -> None:
    """la_stream_probe on raw descriptors."""
    lib = load()
    _raise_on(lib.la_stream_probe(ctypes.byref(desc), stream or None), lib)


def direction_probe_raw(desc: LayerDesc, part: int, begin: int, end: int, fill: int = 0,
                        workgroups_per_cu: int = -1, stream: int = 0) -> None:
    """la_direction_probe on raw descriptors."""
    lib = load()
    _raise_on(lib.la_direction_probe(ctypes.byref(desc), int(part), int(begin), int(end),
                                     int(fill) & 0xFFFFFFFF, int(workgroups_per_cu),
                                     stream or None), lib)


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


def _out_dtype_of(params) -> int:
    import torch
    kinds = {x[3].dtype if len(x) > 3 and x[3] is not None else None for x in params}
    if kinds <= {torch.bfloat16}:
        return OUT_BF16
    if kinds <= {torch.float16}:
        return OUT_FP16
    if kinds == {None}:
        return OUT_NONE
    raise TypeError(f"compute copies must all be bfloat16, all float16 or all None, got {kinds}")


def _describe(params, grads, need_state: bool = True):
    import torch
    if len(params) != len(grads):
        raise ValueError("one list of gradient replicas per tensor")
    if not grads:
        return [], 1, GRAD_BF16, OUT_BF16
    R = len(grads[0])
    if R > MAX_REPLICAS:
        raise ValueError(f"{R} gradient replicas per tensor; at most {MAX_REPLICAS}")
    gd = _grad_dtype_of(grads)
    od = _out_dtype_of(params) if need_state else OUT_NONE
    out = []
    for i, (x, gs) in enumerate(zip(params, grads)):
        n = gs[0].numel() if gs else 0
        d = {"numel": n}
        if need_state:
            p, m, v = x[0], x[1], x[2]
            w = x[3] if len(x) > 3 else None
            n = p.numel()
            d["numel"] = n
            for name, t in (("master", p), ("exp_avg", m), ("exp_avg_sq", v)):
                if t.dtype != torch.float32:
                    raise TypeError(f"tensor {i}: {name} must be float32, got {t.dtype}")
                if t.numel() != n or not t.is_contiguous():
                    raise ValueError(f"tensor {i}: {name} must be a contiguous tensor "
                                     f"of {n} elements")
                d[name] = device_address(t)
            if w is not None:
                if w.numel() != n or not w.is_contiguous():
                    raise ValueError(f"tensor {i}: the compute copy must be a contiguous "
                                     f"tensor of {n} elements")
                d["weight_out"] = device_address(w)
        if len(gs) != R:
            raise ValueError(f"tensor {i}: {len(gs)} gradient replicas, expected {R}")
        for g in gs:
            if g.numel() != n or not g.is_contiguous():
                raise ValueError(f"tensor {i}: gradients must be contiguous tensors "
                                 f"of {n} elements")
        d["grads"] = [device_address(g) for g in gs]
        out.append(d)
    return out, R, gd, od


def _scalar_ptr(t, dtype, what: str) -> int:
    """Address of a one-element (or longer) device scalar of ``dtype`` on the
    current device: the library reads or writes its first element."""
    if not t.is_cuda or t.dtype != dtype:
        raise TypeError(f"{what} must be a {dtype} CUDA tensor, got {t.dtype} on {t.device}")
    if t.numel() < 1:
        raise ValueError(f"{what} has no elements")
    return device_address(t)


def _flag_ptr(flag, what: str = "the flag") -> int:
    import torch
    return 0 if flag is None else _scalar_ptr(flag, torch.int32, what)


def _step_ptr(step_on_device) -> int:
    import torch
    return _scalar_ptr(step_on_device, torch.int64, "step_on_device")


def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def step(params, grads, *, lr: float, beta1: float, beta2: float, eps: float,
         weight_decay: float, step: int, grad_unscale: float = 1.0,
         overflow_flag=None, stream=None) -> None:
    """One LayerAdam update of a layer, enqueued on ``stream`` (default: the
    current torch stream).

    params: per tensor a tuple (master fp32, exp_avg fp32, exp_avg_sq fp32,
            compute copy), updated/written in place; the compute copy is a
            bfloat16 or float16 tensor (the same for every tensor), or None
            for no copy. Every tensor lives in GPU memory or in pinned host
            memory (host-resident state, reached over the host link).
    grads:  per tensor a list of R gradient replicas (all bf16 or all fp16).
    overflow_flag: optional int32 CUDA tensor of one element (set to 1 on a
            non-finite aggregated gradient; never cleared).
    """
    tensors, R, gd, od = _describe(params, grads)
    desc, keep = make_layer(tensors, R, gd, od)
    hp = make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale)
    step_raw(desc, hp, _flag_ptr(overflow_flag), _stream_ptr(stream))
    del keep


def step_range(params, grads, begin: int, end: int, *, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float, step: int, grad_unscale: float = 1.0,
               overflow_flag=None, stream=None) -> None:
    """The update of the layer's elements [begin, end) only (elements
    numbered across the tensors in order)."""
    tensors, R, gd, od = _describe(params, grads)
    desc, keep = make_layer(tensors, R, gd, od)
    hp = make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale)
    step_range_raw(desc, hp, begin, end, _flag_ptr(overflow_flag), _stream_ptr(stream))
    del keep


def step_gated(params, grads, skip_if_nonzero, *, lr: float, beta1: float, beta2: float,
               eps: float, weight_decay: float, step: int, grad_unscale: float = 1.0,
               overflow_flag=None, stream=None) -> None:
    """The update, or nothing at all if the int32 CUDA scalar
    ``skip_if_nonzero`` holds a non-zero value when the kernel runs."""
    tensors, R, gd, od = _describe(params, grads)
    desc, keep = make_layer(tensors, R, gd, od)
    hp = make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale)
    step_gated_raw(desc, hp, _flag_ptr(skip_if_nonzero, "skip_if_nonzero"),
                   _flag_ptr(overflow_flag), _stream_ptr(stream))
    del keep


def step_device_step(params, grads, step_on_device, *, lr: float, beta1: float, beta2: float,
                     eps: float, weight_decay: float, grad_unscale: float = 1.0,
                     overflow_flag=None, stream=None) -> None:
    """The update with t read on the GPU from the int64 CUDA scalar
    ``step_on_device`` when the kernel runs (graph-capturable: advance the
    counter on the device between replays)."""
    t_ptr = _step_ptr(step_on_device)
    tensors, R, gd, od = _describe(params, grads)
    desc, keep = make_layer(tensors, R, gd, od)
    hp = make_params(lr, beta1, beta2, eps, weight_decay, 1, grad_unscale)
    step_device_step_raw(desc, hp, t_ptr, _flag_ptr(overflow_flag), _stream_ptr(stream))
    del keep


def step_ex(params, grads, begin: Optional[int] = None, end: Optional[int] = None, *,
            lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
            step: Optional[int] = None, grad_unscale: float = 1.0, overflow_flag=None,
            skip_if_nonzero=None, step_on_device=None, stream=None) -> None:
    """layer_adam_step_ex: the update with any combination of an element range
    [begin, end), the overflow flag, a device skip flag (int32 CUDA scalar,
    as for step_gated) and a device step count (int64 CUDA scalar, as for
    step_device_step; then ``step`` is not used)."""
    tensors, R, gd, od = _describe(params, grads)
    desc, keep = make_layer(tensors, R, gd, od)
    step_ex_raw(desc, _ex_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale,
                                 step_on_device),
                begin, end, _flag_ptr(overflow_flag),
                _flag_ptr(skip_if_nonzero, "skip_if_nonzero"),
                0 if step_on_device is None else _step_ptr(step_on_device), _stream_ptr(stream))
    del keep


def _ex_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale, step_on_device):
    if step is None and step_on_device is None:
        raise ValueError("give step, or step_on_device")
    return make_params(lr, beta1, beta2, eps, weight_decay, 1 if step is None else step,
                       grad_unscale)


def stream_probe(params, grads, *, stream=None) -> None:
    """la_stream_probe: the update's loads, stores and launch shape without
    its arithmetic (master, m, v rewritten unchanged; the compute copy
    overwritten with the XOR of the replicas) -- a bandwidth measurement."""
    tensors, R, gd, od = _describe(params, grads)
    desc, keep = make_layer(tensors, R, gd, od)
    stream_probe_raw(desc, _stream_ptr(stream))
    del keep


def direction_probe(params, grads, part: int, begin: int = 0, end: Optional[int] = None, *,
                    fill: int = 0, workgroups_per_cu: int = -1, stream=None) -> None:
    """la_direction_probe over the layer's elements [begin, end) (default: all):
    PROBE_READS issues the update's loads only, PROBE_WRITES its stores only
    (master, m, v set to the 32-bit pattern ``fill``, the compute copy to its
    low 16 bits) -- a bandwidth measurement that overwrites the state."""
    tensors, R, gd, od = _describe(params, grads)
    desc, keep = make_layer(tensors, R, gd, od)
    n = sum(t["numel"] for t in tensors)
    direction_probe_raw(desc, part, begin, n if end is None else end, fill, workgroups_per_cu,
                        _stream_ptr(stream))
    del keep


def check_gradients(grads, found_nonfinite, *, grad_unscale: float = 1.0, stream=None) -> None:
    """Set the int32 CUDA scalar ``found_nonfinite`` to 1 if some aggregated
    gradient (sum of the replicas times grad_unscale) is non-finite.
    grads: per tensor a list of R replicas."""
    tensors, R, gd, _ = _describe([None] * len(grads), grads, need_state=False)
    desc, keep = make_layer(tensors, R, gd, OUT_NONE)
    check_gradients_raw(desc, grad_unscale, _flag_ptr(found_nonfinite, "found_nonfinite"),
                        _stream_ptr(stream))
    del keep


class Layer:
    """A layer's buffers described once: every call then passes only the
    hyperparameters and flags (the library still checks all arguments on
    each call). Holds references to the tensors, so they outlive it."""

    def __init__(self, params, grads):
        self._tensors = (list(params), [list(g) for g in grads])
        tensors, self.num_replicas, self.grad_dtype, self.out_dtype = _describe(params, grads)
        self._desc, self._keep = make_layer(tensors, self.num_replicas, self.grad_dtype,
                                            self.out_dtype)
        self.numel = sum(t["numel"] for t in tensors)

    def step(self, *, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
             step: int, grad_unscale: float = 1.0, overflow_flag=None, stream=None) -> None:
        step_raw(self._desc, make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale),
                 _flag_ptr(overflow_flag), _stream_ptr(stream))

    def step_range(self, begin: int, end: int, *, lr: float, beta1: float, beta2: float,
                   eps: float, weight_decay: float, step: int, grad_unscale: float = 1.0,
                   overflow_flag=None, stream=None) -> None:
        step_range_raw(self._desc,
                       make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale),
                       begin, end, _flag_ptr(overflow_flag), _stream_ptr(stream))

    def step_gated(self, skip_if_nonzero, *, lr: float, beta1: float, beta2: float, eps: float,
                   weight_decay: float, step: int, grad_unscale: float = 1.0,
                   overflow_flag=None, stream=None) -> None:
        step_gated_raw(self._desc,
                       make_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale),
                       _flag_ptr(skip_if_nonzero, "skip_if_nonzero"), _flag_ptr(overflow_flag),
                       _stream_ptr(stream))

    def step_device_step(self, step_on_device, *, lr: float, beta1: float, beta2: float,
                         eps: float, weight_decay: float, grad_unscale: float = 1.0,
                         overflow_flag=None, stream=None) -> None:
        step_device_step_raw(self._desc,
                             make_params(lr, beta1, beta2, eps, weight_decay, 1, grad_unscale),
                             _step_ptr(step_on_device), _flag_ptr(overflow_flag),
                             _stream_ptr(stream))

    def step_ex(self, begin: Optional[int] = None, end: Optional[int] = None, *, lr: float,
                beta1: float, beta2: float, eps: float, weight_decay: float,
                step: Optional[int] = None, grad_unscale: float = 1.0, overflow_flag=None,
                skip_if_nonzero=None, step_on_device=None, stream=None) -> None:
        step_ex_raw(self._desc,
                    _ex_params(lr, beta1, beta2, eps, weight_decay, step, grad_unscale,
                               step_on_device),
                    begin, end, _flag_ptr(overflow_flag),
                    _flag_ptr(skip_if_nonzero, "skip_if_nonzero"),
                    0 if step_on_device is None else _step_ptr(step_on_device),
                    _stream_ptr(stream))

    def check_gradients(self, found_nonfinite, *, grad_unscale: float = 1.0,
                        stream=None) -> None:
        check_gradients_raw(self._desc, grad_unscale,
                            _flag_ptr(found_nonfinite, "found_nonfinite"), _stream_ptr(stream))

    def stream_probe(self, stream=None) -> None:
        stream_probe_raw(self._desc, _stream_ptr(stream))

    def direction_probe(self, part: int, begin: int = 0, end: Optional[int] = None, *,
                        fill: int = 0, workgroups_per_cu: int = -1, stream=None) -> None:
        direction_probe_raw(self._desc, part, begin, self.numel if end is None else end, fill,
                            workgroups_per_cu, _stream_ptr(stream))

    def state_bytes(self) -> int:
        return state_bytes_raw(self._desc)

    def traffic_bytes(self) -> int:
        return traffic_bytes_raw(self._desc)


def copy_reference(dst, src, stream=None) -> None:
    """la_copy_reference: copy the bytes of contiguous tensor src into dst
    (same size, a multiple of 16 bytes) with the update's access style -- a
    bandwidth reference, not part of the update."""
    if src.nbytes != dst.nbytes:
        raise ValueError(f"src has {src.nbytes} bytes, dst {dst.nbytes}")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    lib = load()
    _raise_on(lib.la_copy_reference(device_address(dst), device_address(src), src.nbytes,
                                    _stream_ptr(stream) or None), lib)


def state_bytes(numels: Sequence[int], num_replicas: int = 1) -> int:
    """16 bytes per parameter (la_state_bytes)."""
    desc, keep = make_layer([dict(numel=n) for n in numels], num_replicas, GRAD_BF16)
    return state_bytes_raw(desc)


def traffic_bytes(numels: Sequence[int], num_replicas: int, out_dtype: int = OUT_BF16) -> int:
    """(2R + 26) bytes per parameter, (2R + 24) without a compute copy
    (la_traffic_bytes)."""
    desc, keep = make_layer([dict(numel=n) for n in numels], num_replicas, GRAD_BF16, out_dtype)
    return traffic_bytes_raw(desc)
