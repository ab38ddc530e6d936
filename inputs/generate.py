"""Seeded synthetic inputs for the zero-computation-expert MoE layer.

This module draws random numbers and rounds them to the storage types; it holds none of
the layer's arithmetic.  Both the CPU oracle and the GPU library receive exactly the
bits produced here.

Routing inputs (x, W_r, b) are drawn on the host with numpy's PCG64 so that any process
can rebuild them bit for bit; each draw has its own SeedSequence key
(workload seed words, tag, index).  Expert weights, the bulk of the bytes (38.7 GB for
the prefill layer), are drawn with torch's generator on the device that will hold them,
one expert at a time from one seeded generator per tensor; a CPU oracle that needs them
copies the device tensors back.

Storage: fp32 values as float32 arrays; bf16 values as their 16-bit patterns (uint16),
obtained fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest even).

Offline table: workloads whose zero-expert bias shift beta is tuned, and tokens whose
x row is redrawn because two of their top-(K+1) selection scores are too close to order
reliably in fp32, are listed in ``routing_tables.json`` beside this file.  That table is
written by ``oracle/tune_routing_inputs.py``; this module only reads it.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass

import numpy as np

from .configs import Workload

TAG_X, TAG_WR, TAG_B, TAG_WG, TAG_WU, TAG_WD, TAG_PERM, TAG_XR, TAG_DY = range(9)

TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "routing_tables.json")


def rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def seed64(*key) -> int:
    """A 63-bit torch seed derived from a SeedSequence key."""
    s = np.random.SeedSequence([int(k) for k in key]).generate_state(1, np.uint64)[0]
    return int(s) & ((1 << 63) - 1)


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float64).astype(np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def load_table() -> dict:
    if not os.path.exists(TABLE_PATH):
        return {}
    with open(TABLE_PATH) as f:
        return json.load(f)


@dataclass
class RoutingInputs:
    """x [T,d], W_r [E,d] (fp32), b [E] (fp32), exactly as the library receives them."""
    wl: Workload
    x: np.ndarray          # float32 [T,d] (f32 workloads) or uint16 bf16 bits [T,d]
    w_router: np.ndarray   # float32 [E,d]
    bias: np.ndarray       # float32 [E]
    beta: float
    resampled: list
    easy_tokens: np.ndarray
    hard_tokens: np.ndarray

    def x_f64(self) -> np.ndarray:
        if self.wl.dtype == "bf16":
            return bf16_bits_to_f64(self.x)
        return self.x.astype(np.float64)

    def x_torch(self, device):
        import torch
        if self.wl.dtype == "bf16":
            return torch.from_numpy(self.x.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(self.x).to(device)

    def w_router_torch(self, device):
        import torch
        return torch.from_numpy(self.w_router).to(device)

    def bias_torch(self, device):
        import torch
        return torch.from_numpy(self.bias).to(device)


def bias_vector(wl: Workload, beta: float) -> np.ndarray:
    """The fp32 expert-bias vector b [N+Z] of a workload for a given zero-expert shift."""
    N, Z, E = wl.N, wl.Z, wl.E
    kind = wl.bias[0]
    g = rng(*wl.seed_key, TAG_B, 0)
    if kind == "uniform":
        b = g.uniform(-wl.bias[1], wl.bias[1], E)
    elif kind == "uniform+shift":
        b = g.uniform(-wl.bias[1], wl.bias[1], E)
        b[N:] += beta
    elif kind == "exclude_zero":
        b = g.uniform(-wl.bias[1], wl.bias[1], E)
        b[N:] = -2.0
    elif kind == "zipf+shift":
        s, c, a = wl.bias[1], wl.bias[2], wl.bias[3]
        ranks = rng(*wl.seed_key, TAG_PERM, 0).permutation(N) + 1
        b = np.empty(E)
        b[:N] = c * ranks.astype(np.float64) ** (-s)
        b[N:] = beta + g.uniform(-a, a, Z)
    else:
        raise ValueError(f"unknown bias recipe {kind}")
    return b.astype(np.float32)


def routing_inputs(wl: Workload, beta: float | None = None, resample=None) -> RoutingInputs:
    """Build x, W_r and b for a workload.

    beta / resample default to the offline table entry for named workloads; pass them
    explicitly for ad-hoc workloads (tests) or while tuning.  ``resample`` is a list of
    (token, attempt) pairs: token t's base row is redrawn from key (.., TAG_XR, t, attempt).
    """
    T, d, N, E = wl.T, wl.d, wl.N, wl.E
    if beta is None or resample is None:
        entry = load_table().get(wl.name)
        if wl.tuned and entry is None and beta is None:
            raise RuntimeError(f"no tuned bias shift for workload {wl.name}; run "
                               "oracle/tune_routing_inputs.py")
        if beta is None:
            beta = entry["beta"] if entry else 0.0
        if resample is None:
            resample = [tuple(r) for r in entry["resample"]] if entry else []
    x = rng(*wl.seed_key, TAG_X, 0).standard_normal((T, d))
    for t, attempt in resample:
        x[t] = rng(*wl.seed_key, TAG_XR, t, attempt).standard_normal(d)
    w_r = (rng(*wl.seed_key, TAG_WR, 0).standard_normal((E, d)) * wl.router_std).astype(np.float32)
    easy = hard = np.zeros(0, dtype=np.int64)
    if wl.plant_frac > 0:
        n = max(1, int(round(wl.plant_frac * T)))
        order = rng(*wl.seed_key, TAG_PERM, 1).permutation(T)
        easy, hard = np.sort(order[:n]), np.sort(order[n:2 * n])
        wr64 = w_r.astype(np.float64)
        x[easy] += wl.plant_scale * wr64[N:].sum(axis=0)
        x[hard] += wl.plant_scale * wr64[:N].sum(axis=0)
    if wl.dtype == "bf16":
        xs = f64_to_bf16_bits(x)
    else:
        xs = x.astype(np.float32)
    return RoutingInputs(wl=wl, x=xs, w_router=w_r, bias=bias_vector(wl, beta), beta=float(beta),
                         resampled=list(resample), easy_tokens=easy, hard_tokens=hard)


def expert_weights(wl: Workload, device="cpu") -> dict:
    """W_gate [N,I,d], W_up [N,I,d], W_down [N,d,I] as torch tensors on ``device``.

    Each tensor comes from one torch generator seeded from (the workload's weight seed
    words, tag); experts are drawn one after another (fp32 standard normal, times the
    workload's std, rounded to the storage dtype with round-to-nearest-even).  Draws
    depend on the device type.  Workloads with the same weight seed words and shapes (the
    prefill layer and its decode steps) get the same weights.
    """
    import torch
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    out = {}
    for tag, name, shape in ((TAG_WG, "gate", (wl.I, wl.d)), (TAG_WU, "up", (wl.I, wl.d)),
                             (TAG_WD, "down", (wl.d, wl.I))):
        w = torch.empty((wl.N,) + shape, dtype=tdt, device=device)
        g = torch.Generator(device=device)
        g.manual_seed(seed64(*wl.weight_seed_key, tag))
        for e in range(wl.N):
            r = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            w[e].copy_((r * wl.expert_std).to(tdt))
        out[name] = w
    return out


def upstream_grad(wl: Workload) -> np.ndarray:
    """A seeded gradient dy [T,d] of the layer output for the backward: standard normal,
    stored like x (bf16 bits for bf16 workloads, float32 otherwise)."""
    g = rng(*wl.seed_key, TAG_DY, 0).standard_normal((wl.T, wl.d))
    return f64_to_bf16_bits(g) if wl.dtype == "bf16" else g.astype(np.float32)


def weights_f64(t) -> np.ndarray:
    """Exact fp64 copy of a (cpu or device) fp32/bf16 torch tensor, for the oracle."""
    import torch
    return t.detach().cpu().to(torch.float64).numpy()
