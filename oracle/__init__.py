"""Python access to the LayerAdam CPU oracle (``la_oracle.c``).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this package. It loads ``libla_oracle.so`` (built by
gcc from ``la_oracle.c`` alone) through ctypes; it never touches the HIP
library or the GPU.

What the oracle computes, and which passages of the pages each step follows,
is described in ``la_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libla_oracle.so")
# The mutation tests point this at deliberately broken builds of la_oracle.c.
_LIB_OVERRIDE = os.environ.get("LA_ORACLE_LIB_OVERRIDE")

MAX_REPLICAS = 8
GRAD_DTYPES = {"bf16": 0, "fp16": 1}
OUT_DTYPES = {"bf16": 0, "fp16": 1, "none": 2}

# The flags matter for the result: no contraction of a*b+c into a fused
# multiply-add, no fast-math, default x86-64 SSE arithmetic (no x87).
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    """Compile libla_oracle.so with gcc (always recompiles)."""
    cmd = ["gcc", *CFLAGS, "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Tensor(ctypes.Structure):
    _fields_ = [
        ("master", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("weight_out", ctypes.c_void_p),
        ("grad", ctypes.c_void_p * MAX_REPLICAS),
        ("numel", ctypes.c_int64),
    ]


class _Scalars(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float)
                for n in ("b1", "c1", "b2", "c2", "alpha", "q", "e", "d", "u")]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    lib.lao_derive_scalars.argtypes = [ctypes.c_double] * 5 + [
        ctypes.c_int64, ctypes.c_double, ctypes.POINTER(_Scalars)]
    lib.lao_derive_scalars.restype = ctypes.c_int
    lib.lao_decode.argtypes = [ctypes.c_uint16, ctypes.c_int]
    lib.lao_decode.restype = ctypes.c_float
    lib.lao_round_bf16.argtypes = [ctypes.c_float]
    lib.lao_round_bf16.restype = ctypes.c_uint16
    lib.lao_step.argtypes = [ctypes.POINTER(_Tensor), ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.c_int] + [ctypes.c_double] * 5 + [
        ctypes.c_int64, ctypes.c_double, ctypes.POINTER(ctypes.c_int32)]
    lib.lao_step.restype = ctypes.c_int
    lib.lao_check_finite.argtypes = [ctypes.POINTER(_Tensor), ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_double]
    lib.lao_check_finite.restype = ctypes.c_int
    lib.lao_round_fp16_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.lao_round_fp16_array.restype = None
    lib.lao_decode_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int]
    lib.lao_decode_array.restype = None
    lib.lao_round_bf16_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int64]
    lib.lao_round_bf16_array.restype = None
    lib.lao_aggregate_array.argtypes = [ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_float,
                                        ctypes.c_void_p, ctypes.c_int64]
    lib.lao_aggregate_array.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(a: np.ndarray, dtype, n: Optional[int] = None, name: str = "") -> None:
    if a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name}: need a contiguous {np.dtype(dtype)} array")
    if n is not None and a.size != n:
        raise ValueError(f"{name}: need {n} elements, got {a.size}")


def derive_scalars(lr, beta1, beta2, eps, weight_decay, step, unscale=1.0) -> dict:
    s = _Scalars()
    rc = _load().lao_derive_scalars(lr, beta1, beta2, eps, weight_decay, step,
                                    unscale, ctypes.byref(s))
    if rc != 0:
        raise ValueError("oracle: hyperparameters outside their domain")
    return {n: getattr(s, n) for n, _ in _Scalars._fields_}


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    _load().lao_decode_array(_ptr(bits), _ptr(out), bits.size, GRAD_DTYPES[dtype])
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().lao_round_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def round_fp16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().lao_round_fp16_array(_ptr(x), _ptr(out), x.size)
    return out


def aggregate(grads: Sequence[np.ndarray], dtype: str, unscale: float = 1.0) -> np.ndarray:
    grads = [np.ascontiguousarray(g, dtype=np.uint16) for g in grads]
    n = grads[0].size
    for g in grads:
        _check(g, np.uint16, n, "grad")
    ptrs = (ctypes.c_void_p * len(grads))(*[_ptr(g) for g in grads])
    out = np.empty(n, np.float32)
    u = np.float32(unscale)
    _load().lao_aggregate_array(ptrs, len(grads), GRAD_DTYPES[dtype], float(u),
                                _ptr(out), n)
    return out


@dataclass
class Tensor:
    """One tensor of a layer: FP32 master/m/v (updated in place), the
    compute-copy output (BF16 or FP16 bit patterns, written) and the R
    gradient replicas (uint16 bit patterns)."""
    master: np.ndarray
    exp_avg: np.ndarray
    exp_avg_sq: np.ndarray
    weight_out: np.ndarray
    grads: List[np.ndarray] = field(default_factory=list)

    @property
    def numel(self) -> int:
        return self.master.size


def _table(tensors: Sequence[Tensor], need_out: bool):
    replicas = len(tensors[0].grads)
    arr = (_Tensor * len(tensors))()
    for i, t in enumerate(tensors):
        n = t.numel
        _check(t.master, np.float32, n, "master")
        _check(t.exp_avg, np.float32, n, "exp_avg")
        _check(t.exp_avg_sq, np.float32, n, "exp_avg_sq")
        if need_out:
            _check(t.weight_out, np.uint16, n, "weight_out")
            arr[i].weight_out = _ptr(t.weight_out)
        if len(t.grads) != replicas:
            raise ValueError("oracle: every tensor needs the same R")
        arr[i].master = _ptr(t.master)
        arr[i].exp_avg = _ptr(t.exp_avg)
        arr[i].exp_avg_sq = _ptr(t.exp_avg_sq)
        for r, g in enumerate(t.grads):
            _check(g, np.uint16, n, f"grad[{r}]")
            arr[i].grad[r] = _ptr(g)
        arr[i].numel = n
    return arr, replicas


def step(tensors: Sequence[Tensor], *, dtype: str, lr: float, beta1: float,
         beta2: float, eps: float, weight_decay: float, step: int,
         unscale: float = 1.0, with_flag: bool = False,
         out_dtype: str = "bf16") -> Optional[int]:
    """Run one oracle update over ``tensors`` in place. The compute copy goes
    to each tensor's ``weight_out`` array in ``out_dtype`` ("bf16", "fp16"
    or "none"). Returns the overflow flag (0/1) when ``with_flag`` is set."""
    if not tensors:
        raise ValueError("oracle.step: no tensors")
    arr, replicas = _table(tensors, out_dtype != "none")
    flag = ctypes.c_int32(0)
    rc = _load().lao_step(arr, len(tensors), replicas, GRAD_DTYPES[dtype],
                          OUT_DTYPES[out_dtype], lr, beta1, beta2, eps, weight_decay,
                          step, unscale, ctypes.byref(flag) if with_flag else None)
    if rc != 0:
        raise ValueError("oracle.step: invalid arguments")
    return int(flag.value) if with_flag else None


def check_finite(tensors: Sequence[Tensor], *, dtype: str, unscale: float = 1.0) -> int:
    """1 if some aggregated gradient element is +-Inf or NaN, else 0."""
    arr, replicas = _table(tensors, False)
    rc = _load().lao_check_finite(arr, len(tensors), replicas, GRAD_DTYPES[dtype], unscale)
    if rc < 0:
        raise ValueError("oracle.check_finite: invalid arguments")
    return rc
