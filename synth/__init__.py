"""Seeded synthetic LayerAdam inputs (host arrays).

The only module that both sides of a comparison share: it draws the inputs
and holds none of the update's arithmetic. ``libla_synth.so`` is built by gcc
from ``la_synth.c``; see that file for the generator's definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace  # noqa: F401  (replace: Workload variants)
from typing import List, Optional

import numpy as np

from .configs import BENCH_WORKLOAD, HYPER, WORKLOADS, Workload, shrink  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_synth.c")
_LIB_PATH = os.path.join(_HERE, "libla_synth.so")

# per-tensor stream ids: tensor_index * 64 + role
ROLE_MASTER, ROLE_M, ROLE_V, ROLE_SCALE = 0, 1, 2, 3
ROLE_GRAD, ROLE_OUTLIER = 8, 24      # + replica index
GRAD_ALIGN = 8                       # elements between tensor views


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-pthread", "-o",
           _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl, vp, ci = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                 ctypes.c_void_p, ctypes.c_int)
        lib.las_fill_normal_f32.argtypes = [u64, u64, vp, i64, dbl, dbl, ci]
        lib.las_fill_uniform_f32.argtypes = [u64, u64, vp, i64, dbl, dbl, ci]
        lib.las_fill_normal_half.argtypes = [u64, u64, vp, i64, dbl, dbl, u64, dbl,
                                             dbl, ci, ci]
        lib.las_uniform_at.argtypes = [u64, u64, i64]
        lib.las_uniform_at.restype = dbl
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0,
               out: Optional[np.ndarray] = None, threads: Optional[int] = None) -> np.ndarray:
    out = np.empty(n, np.float32) if out is None else out
    _load().las_fill_normal_f32(seed, stream, out.ctypes.data, n, mean, std,
                                threads or default_threads())
    return out


def uniform_f32(seed: int, stream: int, n: int, lo: float = 0.0, hi: float = 1.0,
                out: Optional[np.ndarray] = None, threads: Optional[int] = None) -> np.ndarray:
    out = np.empty(n, np.float32) if out is None else out
    _load().las_fill_uniform_f32(seed, stream, out.ctypes.data, n, lo, hi,
                                 threads or default_threads())
    return out


def normal_half(seed: int, stream: int, n: int, std: float, fmt: str, scale: float = 1.0,
                outlier_stream: int = 0, outlier_prob: float = 0.0,
                outlier_mult: float = 1.0, out: Optional[np.ndarray] = None,
                threads: Optional[int] = None) -> np.ndarray:
    """N(0, std) * scale as BF16/FP16 bit patterns (uint16), rounded toward
    zero; with probability ``outlier_prob`` an element is multiplied by
    ``outlier_mult`` (in FP32) first."""
    out = np.empty(n, np.uint16) if out is None else out
    _load().las_fill_normal_half(seed, stream, out.ctypes.data, n, std, scale,
                                 outlier_stream, outlier_prob, outlier_mult,
                                 1 if fmt == "fp16" else 0, threads or default_threads())
    return out


def uniform_at(seed: int, stream: int, i: int) -> float:
    return _load().las_uniform_at(seed, stream, i)


@dataclass
class LayerInputs:
    """Host arrays of one workload. ``master``, ``exp_avg``, ``exp_avg_sq``
    hold one array per tensor; each gradient replica is one flat per-layer
    buffer (``grad_flat[r]``), with tensor i at element ``grad_offsets[i]``
    (a multiple of 8)."""
    workload: Workload
    master: List[np.ndarray]
    exp_avg: List[np.ndarray]
    exp_avg_sq: List[np.ndarray]
    grad_flat: List[np.ndarray]
    grad_offsets: List[int]
    grad_scales: List[float]

    def grad(self, r: int, i: int) -> np.ndarray:
        off = self.grad_offsets[i]
        return self.grad_flat[r][off:off + self.workload.tensors[i][1]]


def grad_layout(w: Workload):
    offsets, pos = [], 0
    for _, n in w.tensors:
        offsets.append(pos)
        pos += (n + GRAD_ALIGN - 1) // GRAD_ALIGN * GRAD_ALIGN
    return offsets, pos


def make_layer(w: Workload, threads: Optional[int] = None) -> LayerInputs:
    """Draw every input of workload ``w`` (deterministic in its seed)."""
    th = threads or default_threads()
    seed = w.seed
    master, m, v, scales = [], [], [], []
    offsets, total = grad_layout(w)
    grad_flat = [np.zeros(total, np.uint16) for _ in range(w.replicas)]
    for i, (_, n) in enumerate(w.tensors):
        base = i * 64
        master.append(normal_f32(seed, base + ROLE_MASTER, n, 0.0, w.master_std, threads=th))
        if w.m_std is None:
            m.append(np.zeros(n, np.float32))
        else:
            m.append(normal_f32(seed, base + ROLE_M, n, 0.0, w.m_std, threads=th))
        if w.v_high is None:
            v.append(np.zeros(n, np.float32))
        else:
            v.append(uniform_f32(seed, base + ROLE_V, n, 0.0, w.v_high, threads=th))
        scale = w.grad_prescale
        if w.log_scale_range is not None:
            lo, hi = w.log_scale_range
            scale *= 10.0 ** (lo + (hi - lo) * uniform_at(seed, base + ROLE_SCALE, 0))
        scales.append(scale)
        for r in range(w.replicas):
            view = grad_flat[r][offsets[i]:offsets[i] + n]
            normal_half(seed, base + ROLE_GRAD + r, n, w.grad_std, w.grad_dtype,
                        scale=scale, outlier_stream=base + ROLE_OUTLIER + r,
                        outlier_prob=w.outlier_prob, outlier_mult=w.outlier_mult,
                        out=view, threads=th)
    return LayerInputs(w, master, m, v, grad_flat, offsets, scales)
