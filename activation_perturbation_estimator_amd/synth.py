"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds none of the estimator's arithmetic: it only draws the input
arrays (cached logits, targets, layer inputs, caller-side loss changes) that
both the GPU path and the CPU oracle consume.  The pages train on FineWeb with
a 4096-token BPE vocabulary, batches of 8 sequences x 2048 tokens and width 512
(linlog explainer, experiment setup; paper digest, section 3.1); no dataset or
trained weights are available, so these arrays stand in for them.

Recipes (numpy PCG64 `default_rng`, one generator per workload, drawn in the
order targets, logits, X; bf16 rounding is round-to-nearest-even via torch):
  tiny   T=256 (2 x 128), V=512, d=64, K=16, sigma=0.05, gamma=0.
         targets uniform in [0,V); logits fp32 N(0,1); X fp32 N(0,1/d).
  paper  T=16384 (8 x 2048), V=4096, d=512, K=64, sigma=0.02, gamma=0.
         targets Zipf(1.1) over V by inverse CDF (P(k) ~ (k+1)^-1.1, id 0 most
         frequent); logits N(0, variance 2) with +3 on the target logit, then
         bf16; X N(0, 1/512) then bf16.
  k1024  as paper with K=1024.     k16384  as paper with K=16384.
  linear X as paper (bf16 [16384,512]); N=2048, K=256, sigma=0.01, gamma=0.9,
         seq_len 2048; c[K,T] fp32 N(0, variance 1e-3) from default_rng(7).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass
class Workload:
    name: str
    T: int
    seq_len: int
    V: int              # output width N (vocabulary for the head)
    d: int              # input width
    K: int
    sigma: float
    gamma: float
    bf16: bool
    kind: str = "head"  # "head" or "linear"
    data_seed: int = 1
    c_seed: int = 7
    philox_seed: int = 1
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 256, 128, 512, 64, 16, 0.05, 0.0, False),
    "paper": Workload("paper", 16384, 2048, 4096, 512, 64, 0.02, 0.0, True),
    "k1024": Workload("k1024", 16384, 2048, 4096, 512, 1024, 0.02, 0.0, True),
    "linear": Workload("linear", 16384, 2048, 2048, 512, 256, 0.01, 0.9, True, kind="linear"),
    "k16384": Workload("k16384", 16384, 2048, 4096, 512, 16384, 0.02, 0.0, True),
}


def zipf_targets(rng: np.random.Generator, T: int, V: int, s: float = 1.1) -> np.ndarray:
    """T ids in [0,V) with P(k) proportional to (k+1)^-s, by inverse CDF."""
    w = (np.arange(1, V + 1, dtype=np.float64)) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(T)
    return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int32)


def _bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def head_inputs(T: int, V: int, d: int, *, seed: int = 1, bf16: bool = False,
                zipf: bool = False, logit_var: float = 1.0, target_boost: float = 0.0,
                x_var: Optional[float] = None):
    """(logits [T,V], targets [T] int32, X [T,d]) as CPU torch tensors."""
    import torch
    rng = np.random.default_rng(seed)
    y = zipf_targets(rng, T, V) if zipf else rng.integers(0, V, T).astype(np.int32)
    z = rng.standard_normal((T, V), dtype=np.float32) * np.float32(np.sqrt(logit_var))
    if target_boost:
        z[np.arange(T), y] += np.float32(target_boost)
    xv = (1.0 / d) if x_var is None else x_var
    X = rng.standard_normal((T, d), dtype=np.float32) * np.float32(np.sqrt(xv))
    conv = _bf16 if bf16 else _f32
    return conv(z), torch.from_numpy(y), conv(X)


def linear_inputs(T: int, d_in: int, K: int, *, seed: int = 1, c_seed: int = 7,
                  bf16: bool = True, c_var: float = 1e-3):
    """(X [T,d_in], c [K,T] fp32) as CPU torch tensors."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d_in), dtype=np.float32) * np.float32(np.sqrt(1.0 / d_in))
    crng = np.random.default_rng(c_seed)
    c = crng.standard_normal((K, T), dtype=np.float32) * np.float32(np.sqrt(c_var))
    return (_bf16(X) if bf16 else _f32(X)), _f32(c)


def workload_inputs(w: Workload):
    """Inputs of a named workload (see the module docstring for the recipes)."""
    if w.kind == "linear":
        return linear_inputs(w.T, w.d, w.K, seed=w.data_seed, c_seed=w.c_seed, bf16=w.bf16)
    if w.name == "tiny":
        return head_inputs(w.T, w.V, w.d, seed=w.data_seed, bf16=False)
    return head_inputs(w.T, w.V, w.d, seed=w.data_seed, bf16=w.bf16, zipf=True, logit_var=2.0,
                       target_boost=3.0, x_var=1.0 / w.d)


def to_f64(t) -> np.ndarray:
    """Exact promotion of a CPU torch tensor (f32 or bf16) to a float64 array."""
    import torch
    return t.to(torch.float64).numpy()
