"""Seeded synthetic inputs for the attention path (shared by tests, smoke and bench).

This module only draws random numbers and picks shapes; it holds none of the attention
arithmetic, so both the CPU oracle and the HIP path can take their inputs from it.

The shapes follow the model-size table (Table 1) of the CS336 Assignment 2 (systems) handout,
§2.1: head dim = d_model / heads = 64, 64, 64, 80, 128; batch 4 and random data as in its
end-to-end benchmarking setup. The pages use random data, not a dataset.

Recipe: ``torch.Generator('cpu').manual_seed(seed)``, then ``torch.randn`` of shape
``[B, H, N, d]`` in float32 for Q, K, V, dO in that order; bf16 workloads round those values to
bf16 (round to nearest even). ``kv_len`` (key padding) is ``N - floor(N * pad_frac)`` for every
batch row, int32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "kv_len_for"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16": the type of Q, K, V, dO, O and the gradients
    causal: bool = True
    pad_frac: float = 0.0  # fraction of trailing keys masked per batch row
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads, named by what they are.
WORKLOADS = {
    "tiny-f32": Workload("tiny-f32", 1, 2, 128, 64, "f32", True, 0.0, 1),
    "gpt2-small": Workload("gpt2-small", 4, 12, 512, 64, "bf16", True, 0.0, 2),
    "large-4k": Workload("large-4k", 4, 20, 4096, 64, "bf16", True, 0.0, 3),
    "xl-d80-pad": Workload("xl-d80-pad", 4, 32, 2048, 80, "bf16", True, 0.1, 4),
    "10b-16k": Workload("10b-16k", 1, 36, 16384, 128, "bf16", True, 0.0, 5),
}


def kv_len_for(N: int, pad_frac: float) -> int:
    """Unmasked key count when the last ``pad_frac`` of keys is masked: ``N - floor(N*pad_frac)``."""
    return N - int(math.floor(N * pad_frac + 1e-9))


_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = 0,
                pad_frac: float = 0.0, kv_len=None):
    """Return a dict of CPU tensors ``q, k, v, do`` ([B,H,N,d], ``dtype``) and ``kv_len``.

    ``kv_len``: None (no padding) unless ``pad_frac > 0`` or an explicit list/int is given.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    shape = (B, H, N, d)
    out = {}
    for name in ("q", "k", "v", "do"):
        t = torch.randn(shape, dtype=torch.float32, generator=g)
        out[name] = t.to(_TORCH_DTYPE[dtype])
    if kv_len is None and pad_frac > 0:
        kv_len = [kv_len_for(N, pad_frac)] * B
    elif isinstance(kv_len, int):
        kv_len = [kv_len] * B
    out["kv_len"] = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32)
    return out


def make_workload_inputs(w: Workload, seed: int | None = None):
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed if seed is None else seed, w.pad_frac)
