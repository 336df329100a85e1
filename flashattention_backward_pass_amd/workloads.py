"""Seeded synthetic workloads: shapes, value distributions and input generators.

This module holds no attention arithmetic.  It is the only code that both the
HIP path (through tests and bench) and the fp64 oracle consume: it draws Q, K,
V and dO on the CPU from a fixed seed and rounds them to the workload dtype.

Recipe (the same for every workload): a ``torch.Generator`` seeded with the
workload's seed draws, in this order, Q [B,H,N,d], K [B,H_kv,N,d],
V [B,H_kv,N,d] and dO [B,H,N,d] as iid normal float32 values; Q and K are
scaled by ``sigma_qk``; all four are then rounded to the workload dtype (bf16
rounding is round-to-nearest-even).  O and LSE are not drawn: they come from
the forward pass on these inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    H_kv: int
    N: int
    d: int
    dtype: str          # "fp32" or "bf16"
    causal: bool
    softcap: float      # 0 = no cap; c > 0 caps the raw scores as c * tanh(QK^T / c)
    tau: float          # softmax scale
    sigma_qk: float     # standard deviation of Q and K entries (V and dO: 1)
    seed: int
    window: tuple = (-1, -1)  # local mask (window_left, window_right); -1 = unbounded side
    dropout: tuple = None     # (p, seed, offset) of the dropout mask, or None

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def group(self) -> int:
        return self.H // self.H_kv

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs of one head that the masks leave visible."""
        import numpy as np
        n = self.N
        i = np.arange(n, dtype=np.int64)
        wl, wr = self.window
        lo = np.maximum(0, i - wl) if wl >= 0 else np.zeros(n, dtype=np.int64)
        hi = np.full(n, n - 1, dtype=np.int64)
        if wr >= 0:
            hi = np.minimum(hi, i + wr)
        if self.causal:
            hi = np.minimum(hi, i)
        return int(np.maximum(hi - lo + 1, 0).sum())

    def flops(self) -> float:
        """Backward FLOPs of the metric: 10 N^2 d per query head, halved when causal.
        With a local window: 10 d per visible (query, key) pair."""
        if tuple(self.window) != (-1, -1):
            return 10.0 * self.B * self.H * self.d * self.visible_pairs()
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def asdict(self):
        return asdict(self)


def _wl(name, B, H, H_kv, N, d, dtype, causal, softcap, sigma_qk, seed, window=(-1, -1), dropout=None):
    return Workload(name, B, H, H_kv, N, d, dtype, causal, softcap, 1.0 / math.sqrt(d), sigma_qk, seed, window,
                    dropout)


# The workloads of the parity and performance suite.
WORKLOADS = {
    w.name: w
    for w in [
        _wl("fp32_b1h1_n128_d64", 1, 1, 1, 128, 64, "fp32", False, 0.0, 1.0, 1000),
        _wl("bf16_causal_b2h16_n1024_d64", 2, 16, 16, 1024, 64, "bf16", True, 0.0, 1.0, 1001),
        _wl("bf16_softcap30_b4h16_n2048_d128", 4, 16, 16, 2048, 128, "bf16", False, 30.0, 1.5, 1002),
        _wl("bf16_gqa32x8_causal_b1_n4096_d128", 1, 32, 8, 4096, 128, "bf16", True, 0.0, 1.0, 1003),
        _wl("bf16_causal_b1h8_n16384_d128", 1, 8, 8, 16384, 128, "bf16", True, 0.0, 1.0, 1004),
        # Local (sliding-window) variant of the long workload: each query sees
        # itself and the 2048 keys before it.
        _wl("bf16_local2048_causal_b1h8_n16384_d128", 1, 8, 8, 16384, 128, "bf16", True, 0.0, 1.0, 1005,
            (2048, -1)),
        # Dropout variant of the long workload: p = 0.1, generator seed and
        # offset fixed.
        _wl("bf16_dropout0.1_causal_b1h8_n16384_d128", 1, 8, 8, 16384, 128, "bf16", True, 0.0, 1.0, 1006,
            dropout=(0.1, 0x5EED0000_00001006, 0)),
        # One GPU's share of the long workload sharded by heads over 8 GPUs:
        # a single head at its full length.
        _wl("bf16_causal_b1h1_n16384_d128", 1, 1, 1, 16384, 128, "bf16", True, 0.0, 1.0, 1007),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)


def custom(B, H, H_kv, N, d, dtype="bf16", causal=False, softcap=0.0, tau=None, sigma_qk=1.0, seed=0,
           name="custom", window=(-1, -1), dropout=None) -> Workload:
    """A workload of any shape, for edge-case tests (ragged N, tiny sizes, ...)."""
    return Workload(name, B, H, H_kv, N, d, dtype, causal, float(softcap),
                    float(tau) if tau is not None else 1.0 / math.sqrt(d), sigma_qk, seed, tuple(window),
                    tuple(dropout) if dropout is not None else None)


def make_inputs(w: Workload):
    """Seeded CPU tensors Q, K, V, dO of the workload dtype (see module docstring)."""
    g = torch.Generator().manual_seed(w.seed)
    f32 = torch.float32
    Q = torch.randn(w.B, w.H, w.N, w.d, generator=g, dtype=f32) * w.sigma_qk
    K = torch.randn(w.B, w.H_kv, w.N, w.d, generator=g, dtype=f32) * w.sigma_qk
    V = torch.randn(w.B, w.H_kv, w.N, w.d, generator=g, dtype=f32)
    dO = torch.randn(w.B, w.H, w.N, w.d, generator=g, dtype=f32)
    dt = w.torch_dtype
    return {"Q": Q.to(dt), "K": K.to(dt), "V": V.to(dt), "dO": dO.to(dt)}
