"""Shared pieces of the GPU tests: upload seeded inputs, run the HIP path
through the C ABI, run the oracle on the same inputs, compare.

Comparison rule: master, m and v within 2 FP32 ulp (ordered-integer distance,
+0 and -0 equal, NaN only against NaN); the compute copy bit-exact, both against
the oracle's RNE cast of the GPU's own master and against the oracle's BF16.
"""
from __future__ import annotations

import sys
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import optimizer_step_layeradam_amd as la
import oracle
import synth

ULP_TOL = 2


# Tensor sizes of the ragged layers: single elements, the short entries that
# may start unaligned, both sides of the update's 256-element chunk and of
# two chunks, of the 2048- and 4096-element powers of two (4096: the finite
# check's chunk), and longer tensors with ragged tails.
RAGGED = (("a", 1), ("b", 3), ("c", 7), ("p", 255), ("q", 256), ("r", 257),
          ("j", 511), ("k", 512), ("l", 513),
          ("d", 2047), ("e", 2048), ("f", 2049), ("m", 4095), ("n", 4096), ("o", 4097),
          ("g", 4101), ("h", 10001), ("i", 65536 + 13))


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def ordered(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    d = np.abs(ordered(a) - ordered(b))
    na, nb = np.isnan(a), np.isnan(b)
    d = np.where(na & nb, 0, d)
    d = np.where(na ^ nb, np.iinfo(np.int64).max, d)
    return d


def grad_torch_dtype(w: synth.Workload):
    return torch.float16 if w.grad_dtype == "fp16" else torch.bfloat16


def to_device_u16(a: np.ndarray, dtype, device) -> torch.Tensor:
    return torch.from_numpy(a.view(np.int16)).to(device).view(dtype)


class GpuLayer:
    """One workload's inputs resident on the GPU, laid out as the benchmark
    lays them out: one allocation per master/m/v/BF16 tensor, one flat
    buffer per gradient replica with tensor views at multiples of 8."""

    def __init__(self, L: synth.LayerInputs, device="cuda:0", out: str = "bf16"):
        self.L = L
        self.out = out
        w = L.workload
        dev = torch.device(device)
        gdt = grad_torch_dtype(w)
        self.params = []
        self.out_buffers = []
        odt = {"bf16": torch.bfloat16, "fp16": torch.float16, "none": torch.bfloat16}[out]
        for i, (_, n) in enumerate(w.tensors):
            p = torch.from_numpy(L.master[i]).to(dev)
            m = torch.from_numpy(L.exp_avg[i]).to(dev)
            v = torch.from_numpy(L.exp_avg_sq[i]).to(dev)
            # 0x7FAA: a NaN payload neither cast produces, to spot unwritten elements
            wb = torch.full((n,), 0x7FAA, dtype=torch.int16, device=dev).view(odt)
            self.out_buffers.append(wb)
            self.params.append((p, m, v, None if out == "none" else wb))
        self.grad_flat = [to_device_u16(g, gdt, dev) for g in L.grad_flat]
        self.grads = [[gf[off:off + n] for gf in self.grad_flat]
                      for off, (_, n) in zip(L.grad_offsets, w.tensors)]
        self.flag = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(self, t: Optional[int] = None, with_flag: Optional[bool] = None, **hp_over):
        w = self.L.workload
        hp = dict(w.hyper)
        hp.update(hp_over)
        unscale = hp.pop("unscale", w.unscale)
        use_flag = w.with_flag if with_flag is None else with_flag
        la.step(self.params, self.grads, step=w.step if t is None else t,
                grad_unscale=unscale, overflow_flag=self.flag if use_flag else None, **hp)

    def download(self) -> Dict[str, List[np.ndarray]]:
        torch.cuda.synchronize()
        out = {"master": [], "exp_avg": [], "exp_avg_sq": [], "weight_out": []}
        for (p, m, v, _), wb in zip(self.params, self.out_buffers):
            out["master"].append(p.cpu().numpy())
            out["exp_avg"].append(m.cpu().numpy())
            out["exp_avg_sq"].append(v.cpu().numpy())
            out["weight_out"].append(wb.view(torch.int16).cpu().numpy().view(np.uint16))
        out["flag"] = int(self.flag.item())
        return out

    def free(self):
        self.params = self.grads = self.grad_flat = self.out_buffers = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def oracle_tensors(L: synth.LayerInputs, idx: Optional[Sequence[np.ndarray]] = None):
    w = L.workload
    ts = []
    for i, (_, n) in enumerate(w.tensors):
        sel = slice(None) if idx is None else idx[i]
        g = [np.ascontiguousarray(L.grad(r, i)[sel]) for r in range(w.replicas)]
        p = np.array(L.master[i][sel], np.float32)
        ts.append(oracle.Tensor(p, np.array(L.exp_avg[i][sel], np.float32),
                                np.array(L.exp_avg_sq[i][sel], np.float32),
                                np.zeros(p.size, np.uint16), g))
    return ts


def oracle_step(L: synth.LayerInputs, ts, t: Optional[int] = None,
                with_flag: Optional[bool] = None, out: str = "bf16",
                **hp_over) -> Optional[int]:
    w = L.workload
    hp = dict(w.hyper)
    hp.update(hp_over)
    unscale = hp.pop("unscale", w.unscale)
    use_flag = w.with_flag if with_flag is None else with_flag
    return oracle.step(ts, dtype=w.grad_dtype, step=w.step if t is None else t,
                       unscale=unscale, with_flag=use_flag, out_dtype=out, **hp)


@dataclass
class Report:
    compared: int = 0
    max_ulp: int = 0
    nonzero_ulp: int = 0
    bf16_mismatch: int = 0

    def __str__(self):
        return (f"compared={self.compared} max_ulp={self.max_ulp} "
                f"nonzero_ulp={self.nonzero_ulp} bf16_mismatch={self.bf16_mismatch}")


def compare(gpu: Dict[str, List[np.ndarray]], ts, idx=None, report: Optional[Report] = None,
            label: str = "", out: str = "bf16") -> Report:
    """Compare GPU outputs (whole tensors, or sampled at idx) with oracle
    tensors; assert the parity bar and return statistics. ``out`` is the
    compute-copy format ("bf16", "fp16", or "none": the buffer must still hold
    its 0x7FAA fill)."""
    rep = report or Report()
    for i, x in enumerate(ts):
        sel = slice(None) if idx is None else idx[i]
        for field in ("master", "exp_avg", "exp_avg_sq"):
            g = gpu[field][i][sel]
            o = getattr(x, field)
            d = ulp_distance(g, o)
            worst = int(d.max()) if d.size else 0
            if worst > ULP_TOL:
                j = int(np.argmax(d))
                raise AssertionError(f"{label} tensor {i} {field}[{j}]: gpu={g[j]!r} "
                                     f"oracle={o[j]!r} ({worst} ulp)")
            rep.max_ulp = max(rep.max_ulp, worst)
            rep.nonzero_ulp += int(np.count_nonzero(d))
        gw = gpu["weight_out"][i][sel]
        if out == "none":
            assert np.all(gw == 0x7FAA), f"{label} tensor {i}: compute copy written"
            rep.compared += int(gw.size)
            continue
        # the compute copy is exactly the RNE cast of the GPU's own master ...
        cast = oracle.round_fp16 if out == "fp16" else oracle.round_bf16
        own = cast(gpu["master"][i][sel])
        bad = np.nonzero(gw != own)[0]
        if bad.size:
            j = int(bad[0])
            raise AssertionError(f"{label} tensor {i} weight_out[{j}] = {gw[j]:#06x}, "
                                 f"RNE_{out}(master) = {own[j]:#06x}")
        # ... and equals the oracle's wherever the masters agree bit for bit
        same = gpu["master"][i][sel].view(np.uint32) == x.master.view(np.uint32)
        rep.bf16_mismatch += int(np.count_nonzero((gw != x.weight_out) & same))
        assert rep.bf16_mismatch == 0, f"{label} tensor {i}: copy differs where masters agree"
        rep.compared += int(gw.size)
    return rep


def slices_of(w: synth.Workload, size: int):
    """(tensor, begin, end) for every tensor cut into slices of ``size``."""
    out = []
    for i, (_, n) in enumerate(w.tensors):
        for a in range(0, n, size):
            out.append((i, a, min(n, a + size)))
    return out


def compare_every_element(gl: GpuLayer, L: synth.LayerInputs, slice_size: int = 1 << 24,
                          threads: int = 16, label: str = "", **hp_over):
    """Compare every element of the GPU's state and compute copy after one
    step (already taken on ``gl``) with the oracle run on the same inputs,
    one slice at a time: each worker downloads a slice of master/m/v/copy,
    runs the oracle on the matching input slice and compares, so host memory
    stays bounded by threads x slice. Returns (Report, oracle flag)."""
    w = L.workload
    torch.cuda.synchronize()
    lock = threading.Lock()
    total = Report()
    flags = []

    def one(item):
        i, a, b = item
        p, m, v, _ = gl.params[i]
        wb = gl.out_buffers[i]
        got = {"master": [p[a:b].cpu().numpy()], "exp_avg": [m[a:b].cpu().numpy()],
               "exp_avg_sq": [v[a:b].cpu().numpy()],
               "weight_out": [wb.view(torch.int16)[a:b].cpu().numpy().view(np.uint16)]}
        ts = [oracle.Tensor(np.array(L.master[i][a:b], np.float32),
                            np.array(L.exp_avg[i][a:b], np.float32),
                            np.array(L.exp_avg_sq[i][a:b], np.float32),
                            np.zeros(b - a, np.uint16),
                            [np.ascontiguousarray(L.grad(r, i)[a:b])
                             for r in range(w.replicas)])]
        flag = oracle_step(L, ts, **hp_over)
        rep = compare(got, ts, label=f"{label} tensor {i} [{a}, {b})", out=gl.out)
        with lock:
            total.compared += rep.compared
            total.max_ulp = max(total.max_ulp, rep.max_ulp)
            total.nonzero_ulp += rep.nonzero_ulp
            total.bf16_mismatch += rep.bf16_mismatch
            flags.append(flag or 0)

    with ThreadPoolExecutor(threads) as ex:
        for _ in ex.map(one, slices_of(w, slice_size)):
            pass
    assert total.compared == w.numel, (total.compared, w.numel)
    return total, max(flags) if flags else 0
