"""Seeded synthetic inputs for the Periodic Row-wise Muon step.

Shared by the tests and the benchmark; holds none of the optimizer's
arithmetic (no momentum, no normalisation, no Newton-Schulz), only shapes and
random numbers.  Both the oracle and the HIP library receive the exact values
produced here.

Parameter sets are DiT-shaped: per transformer block of width d the 2-D
weights are qkv (3d x d), proj (d x d), fc1 (4d x d), fc2 (d x 4d) and adaLN
(6d x d), stored PyTorch-style as (out, in) row-major.  The pages train DiTs
from 1.3B to 15B parameters but do not print widths or depths; the sets below
stand in for them.  Weights start from N(0, 0.02^2); gradients are i.i.d.
normal with the stated standard deviation, rounded to nearest-even when they
are stored as bf16.
"""

from __future__ import annotations

import dataclasses

import numpy as np

DEFAULT_SEED = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple            # ((label, m, n), ...)
    grad_dtype: str          # "f32" | "bf16"
    grad_std: float
    steps: int
    overrides: tuple = ()    # ((config_field, value), ...)
    d: int = 0
    blocks: int = 0

    @property
    def elements(self) -> int:
        return sum(m * n for _, m, n in self.shapes)


def dit_block_shapes(d: int):
    return (("qkv", 3 * d, d), ("proj", d, d), ("fc1", 4 * d, d),
            ("fc2", d, 4 * d), ("adaln", 6 * d, d))


def dit_bias_sizes(d: int):
    """Per-block bias lengths of the same block (qkv, proj, fc1, fc2, adaLN)."""
    return (3 * d, d, 4 * d, d, 6 * d)


def _dit(name, d, blocks, steps, overrides=()):
    shapes = tuple((f"b{b}.{lab}", m, n) for b in range(blocks)
                   for lab, m, n in dit_block_shapes(d))
    return Workload(name, shapes, "bf16", 1e-3, steps, tuple(overrides), d, blocks)


WORKLOADS = {
    "single-256x512": Workload("single-256x512", (("w", 256, 512),), "f32", 1.0, 6),
    "dit-1.3b": _dit("dit-1.3b", 2048, 18, 30),
    "dit-4b": _dit("dit-4b", 3072, 24, 30),
    "dit-4b-muonbp": _dit("dit-4b-muonbp", 3072, 24, 30,
                          (("bp_blocks", 8), ("bp_period", 3), ("bp_lr_ratio", 0.5))),
    "dit-15b": _dit("dit-15b", 5120, 32, 12),
}


# ------------------------------------------------------------------ host RNG
def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def host_normal(shape, std: float, dtype: str, *key: int) -> np.ndarray:
    """i.i.d. N(0, std^2) as float32, bf16-representable when dtype is bf16."""
    x = (_rng(*key).standard_normal(shape) * std).astype(np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def host_grad(seed: int, t: int, idx: int, shape, std: float, dtype: str) -> np.ndarray:
    return host_normal(shape, std, dtype, seed, 1, t, idx)


def host_weight0(seed: int, idx: int, shape, std: float = 0.02) -> np.ndarray:
    return host_normal(shape, std, "f32", seed, 2, idx)


SPECTRA = ("geometric-1e-4", "geometric-1e-2", "rank-8th-noise", "one-spike")


def host_spectrum_matrix(seed: int, idx: int, shape, kind: str, scale: float = 1e-2) -> np.ndarray:
    """A float32 matrix U diag(s) V^T with random orthonormal U, V and a set
    spectrum s over the short side r: falling geometrically from 1 to 1e-4 or
    1e-2, r/8 ones plus N(0, 1e-6) noise everywhere, or one value 100 and the
    rest 1.  Momenta of trained networks are far from the flat spectra of
    i.i.d. gradients; these stand in for them."""
    m, n = shape
    r = min(m, n)
    g = _rng(seed, 3, idx, SPECTRA.index(kind))
    u, _ = np.linalg.qr(g.standard_normal((m, r)))
    v, _ = np.linalg.qr(g.standard_normal((n, r)))
    if kind == "geometric-1e-4":
        s = 10.0 ** (-4.0 * np.arange(r) / r)
    elif kind == "geometric-1e-2":
        s = 10.0 ** (-2.0 * np.arange(r) / r)
    elif kind == "rank-8th-noise":
        s = np.r_[np.ones(max(1, r // 8)), np.zeros(r - max(1, r // 8))]
    else:
        s = np.r_[100.0, np.ones(r - 1)]
    x = (u * s) @ v.T
    if kind == "rank-8th-noise":
        x = x + 1e-3 * g.standard_normal((m, n))
    return (x * scale).astype(np.float32)


# ------------------------------------------------------------------ device RNG
def device_normal_(out, std: float, seed: int):
    """Fill a CUDA tensor in place with seeded N(0, std^2) values.

    Uses torch's Philox generator on the device; the values are inputs only.
    """
    import torch
    g = torch.Generator(device=out.device)
    g.manual_seed(int(seed))
    if out.dtype == torch.float32:
        out.normal_(0.0, std, generator=g)
    else:
        tmp = torch.empty(out.shape, dtype=torch.float32, device=out.device)
        tmp.normal_(0.0, std, generator=g)
        out.copy_(tmp)
    return out


def seed_for(seed: int, t: int, idx: int, kind: int = 1) -> int:
    return (int(seed) * 1_000_003 + kind * 7_919 + t * 104_729 + idx * 15_485_863) % (2 ** 62)
