"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic: it only draws random numbers and
rounds them to the storage dtype.  Both the GPU library's callers and the CPU
oracle's callers take their inputs from here, so the two sides see the same
bits.

Recipe (one per workload; q is contiguous [B, H, N, d], k and v are
contiguous [B, H_kv, N_kv, d], which is [B, H, N, d] unless the workload
groups K/V heads or has its own key length):
  * ``numpy.random.default_rng(seed)`` (PCG64), drawn in the order Q, K, V;
  * ``normal``: Q, K, V = standard_normal(float32);
  * ``large_logit``: Q, K = 3 * standard_normal(float32) (scores with a
    standard deviation near 9, so the running max moves a lot and rescaling is
    exercised), V = 2 * random(float32) - 1, i.e. uniform on [-1, 1);
  * the float32 draws are rounded to the workload dtype with round-to-nearest-
    even (torch CPU ``.to``), and those rounded values are the inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" | "bf16" | "f16"
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    dist: str = "normal"
    Hkv: int = 0        # K/V heads (0: same as H)
    Nkv: int = 0        # keys per K/V head (0: same as N, the query rows)
    splits: int = 1     # key ranges fa_fwd_ex uses (0: the library's default)

    @property
    def h_kv(self) -> int:
        return self.Hkv or self.H

    @property
    def n_kv(self) -> int:
        return self.Nkv or self.N

    @property
    def extended(self) -> bool:
        """True when the workload needs fa_fwd_ex rather than fa_fwd."""
        return self.h_kv != self.H or self.n_kv != self.N or self.splits != 1

    @property
    def scale(self) -> float:
        """1/sqrt(d), as the fp32 number the library receives."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Metric FLOPs: 4*B*H*N_q*N_kv*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.n_kv * self.d
        return f / 2.0 if self.causal else f

    @property
    def visible_pairs(self) -> int:
        n, nk = self.N, self.n_kv
        if self.causal:  # query i sees keys j <= i + nk - n
            per_head = sum(max(0, min(nk, i + 1 + nk - n)) for i in range(n)) if n != nk \
                else n * (n + 1) // 2
        else:
            per_head = n * nk
        return self.B * self.H * per_head

    @property
    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O and LSE written once."""
        e = 4 if self.dtype == "f32" else 2
        q = self.B * self.H * self.N * self.d * e
        kv = 2 * self.B * self.h_kv * self.n_kv * self.d * e
        return 2 * q + kv + 4 * self.B * self.H * self.N

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads (plus the ragged variant of the second) that the parity
# tests and the benchmark use, and the shapes of the split-KV / grouped-head
# entry point:
#   C1s  the one-head fp32 workload run with its keys split into 8 ranges;
#   D1   one decoding step: one query row per head against 16384 cached keys,
#        32 query heads sharing 8 K/V heads, head size 128, bf16;
#   G1   the headline bf16 shape with 16 query heads on 4 K/V heads;
#   G2   a causal bf16 prefill with 16 query heads on 2 K/V heads.
WORKLOADS = {
    "C1": Workload("C1", "f32", 1, 1, 512, 64, False, 0),
    "C2": Workload("C2", "f32", 4, 8, 2048, 64, False, 1),
    "C2r": Workload("C2r", "f32", 4, 8, 2000, 64, False, 1),
    "C3": Workload("C3", "bf16", 8, 16, 4096, 128, True, 2),
    "C4": Workload("C4", "bf16", 1, 16, 16384, 64, False, 3),
    "C5": Workload("C5", "f16", 2, 32, 8191, 128, True, 4, "large_logit"),
    "C1s": Workload("C1s", "f32", 1, 1, 512, 64, False, 0, splits=8),
    "D1": Workload("D1", "bf16", 8, 32, 1, 128, False, 5, Hkv=8, Nkv=16384, splits=0),
    "G1": Workload("G1", "bf16", 1, 16, 16384, 64, False, 6, Hkv=4),
    "G2": Workload("G2", "bf16", 8, 16, 4096, 128, True, 7, Hkv=2),
}


def make_inputs(w: Workload):
    """Return (q, k, v) as CPU torch tensors of the workload's dtype."""
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    kv_shape = (w.B, w.h_kv, w.n_kv, w.d)
    if w.dist == "normal":
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(kv_shape, dtype=np.float32)
        v = rng.standard_normal(kv_shape, dtype=np.float32)
    elif w.dist == "large_logit":
        q = 3.0 * rng.standard_normal(shape, dtype=np.float32)
        k = 3.0 * rng.standard_normal(kv_shape, dtype=np.float32)
        v = rng.random(kv_shape, dtype=np.float32) * 2.0 - 1.0
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    tdt = TORCH_DTYPES[w.dtype]
    return tuple(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(tdt)
                 for x in (q, k, v))


def make_upstream(w: Workload, seed: int):
    """A seeded upstream gradient dL/dO: [B, H, N, d] N(0, 1), rounded to the workload's dtype."""
    x = np.random.default_rng(seed).standard_normal((w.B, w.H, w.N, w.d)).astype(np.float32)
    return torch.from_numpy(x).to(TORCH_DTYPES[w.dtype])


def sample_rows(w: Workload, count: int, seed: int = 12345) -> np.ndarray:
    """Deterministic sample of flat row indices (b*H + h)*N + i.

    Always includes the first and last row of the first and last head (the
    causal corner cases and the ragged tail) plus uniformly drawn rows.
    """
    total = w.B * w.H * w.N
    fixed = {0, w.N - 1, max(0, total - w.N), total - 1}
    rng = np.random.default_rng(seed)
    drawn = rng.choice(total, size=min(count, total), replace=False)
    rows = np.array(sorted(fixed.union(int(r) for r in drawn)), dtype=np.int64)
    return rows
