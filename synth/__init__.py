"""Seeded synthetic inputs shared by the CPU oracle and the GPU library.

This module draws random numbers and shapes test data; it contains none of
the quantizer's arithmetic. Both sides of every parity check receive the
same arrays from here:

* the Gaussian matrices the method draws (the matrix whose QR factor is the
  random rotation, and the JL sketch matrix), as float64 host arrays;
* key/value/query vectors with the workloads' shapes and value laws:
  i.i.d. N(0,1), the "outlier-channel" law (N(0,1) scaled per channel by
  lognormal(0,1), four channels further scaled by 20), and unit-norm
  Gaussian vectors for vector search.

Host arrays come from numpy's PCG64 seeded with SeedSequence([seed, *tags]).
Large device-resident inputs come from torch's device generator seeded with a
value derived the same way; tests that check such inputs copy the sampled
rows back to the host before handing them to the oracle.
"""
from __future__ import annotations

import numpy as np

# Stream tags: the Gaussian matrix behind the rotation, the sketch matrix,
# and the data streams.
TAG_ROTATION = 1
TAG_SKETCH = 2
TAG_KEYS = 10
TAG_VALUES = 11
TAG_QUERIES = 12
TAG_SCALES_K = 13
TAG_SCALES_V = 14
TAG_APPEND_K = 15
TAG_APPEND_V = 16
TAG_DB = 17


def rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *[int(t) for t in tags]])))


def torch_seed(seed: int, *tags: int) -> int:
    """A 63-bit seed for torch generators, derived from (seed, tags)."""
    return int(np.random.SeedSequence([int(seed), *[int(t) for t in tags]]).generate_state(2, np.uint64)[0] >> np.uint64(1))


def gaussian_matrix(seed: int, tag: int, rows: int, cols: int) -> np.ndarray:
    """i.i.d. N(0,1) float64 matrix, row-major, for the rotation (tag 1) or sketch (tag 2)."""
    return rng(seed, tag).standard_normal((rows, cols))


def to_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to bfloat16 (round-to-nearest-even), returned as float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32)


def bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    return (np.ascontiguousarray(x_f32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def outlier_scales(seed: int, tag: int, d: int, n_outliers: int = 4, factor: float = 20.0) -> np.ndarray:
    """Per-channel scales: exp(N(0,1)) for every channel, times `factor` on `n_outliers` channels."""
    g = rng(seed, tag)
    s = np.exp(g.standard_normal(d))
    idx = g.choice(d, size=n_outliers, replace=False)
    s[idx] *= factor
    return s


def gaussian(seed: int, tags: tuple, shape: tuple, dtype: str = "f32") -> np.ndarray:
    """N(0,1) values as float32 ("f32") or bf16-rounded float32 ("bf16")."""
    x = rng(seed, *tags).standard_normal(shape).astype(np.float32)
    return to_bf16_f32(x) if dtype == "bf16" else x


def outlier_kv(seed: int, tags: tuple, scale_tag: int, shape: tuple, dtype: str = "bf16") -> np.ndarray:
    """Outlier-channel data: N(0,1) scaled per channel (last axis), rounded to bf16."""
    s = outlier_scales(seed, scale_tag, shape[-1]).astype(np.float32)
    x = rng(seed, *tags).standard_normal(shape).astype(np.float32) * s
    return to_bf16_f32(x) if dtype == "bf16" else x.astype(np.float32)


def unit_gaussian(seed: int, tags: tuple, shape: tuple) -> np.ndarray:
    """Gaussian rows normalized to unit norm, float32."""
    x = rng(seed, *tags).standard_normal(shape)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x.astype(np.float32)


# ----------------------------------------------------------------------------
# Device-side generators for full-size workloads (torch is plumbing here).
# ----------------------------------------------------------------------------

def torch_gaussian(seed: int, tags: tuple, shape: tuple, dtype, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, *tags))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def torch_outlier_kv(seed: int, tags: tuple, scale_tag: int, shape: tuple, dtype, device):
    import torch
    s = torch.from_numpy(outlier_scales(seed, scale_tag, shape[-1]).astype(np.float32)).to(device)
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, *tags))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(s)
    return x.to(dtype)


def torch_unit_gaussian(seed: int, tags: tuple, shape: tuple, device, chunk_rows: int = 1 << 16):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, *tags))
    out = torch.empty(shape, device=device, dtype=torch.float32)
    flat = out.view(-1, shape[-1])
    for i in range(0, flat.shape[0], chunk_rows):
        blk = torch.randn((min(chunk_rows, flat.shape[0] - i), shape[-1]), generator=g, device=device, dtype=torch.float64)
        blk /= blk.norm(dim=1, keepdim=True)
        flat[i:i + blk.shape[0]] = blk.to(torch.float32)
    return out
