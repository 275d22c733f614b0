"""Seeded synthetic inputs with the shapes and value distributions of the codec's workloads.

This module holds no step of the codec: it only draws numbers.  Both the GPU tests/benchmark and
the CPU oracle tests take their inputs from here.  Everything is drawn on the host with numpy's
PCG64 generator and rounded to bfloat16 (round to nearest even) where the workload is bf16, so the
same host array feeds the GPU and the oracle.

Workloads (the HyperQuant summaries evaluate on Llama-3.1-8B weights and KV caches; no checkpoint
or dataset is used here -- these random tensors take the 8B model's shapes instead):

* ``tiny``   64 x 128 fp32 N(0,1); 1% of the coordinates (82 positions, without replacement) x20.
* ``weight`` 14336 x 4096 bf16 N(0, 0.02^2) (an MLP projection, input dim 4096, tiles of 128
  along it); round(0.005 * 4096) = 20 input columns, without replacement, replaced by
  0.02 * 5 * t, t ~ Student-t(4).
* ``kv``     per (layer, K|V) call a [8 kv heads][32768 tokens][128] bf16 N(0,1) tensor; for K,
  4 channels per (layer, head), fixed for the whole cache, are scaled x10.
* ``model``  the 224 linear weights of an 8B-shaped decoder (32 layers of q, k, v, o, gate, up,
  down) N(0, 0.02^2) bf16, generated one tensor at a time.
"""
from __future__ import annotations

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    flat = u.reshape(-1)
    step = 1 << 22
    for i in range(0, flat.size, step):
        blk = flat[i:i + step]
        lsb = (blk >> 16) & np.uint32(1)
        blk += np.uint32(0x7FFF)
        blk += lsb
        blk >>= 16
    return u.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def tiny(seed: int = 0, tiles: int = 64) -> np.ndarray:
    g = _rng(seed)
    x = g.standard_normal(tiles * 128, dtype=np.float32)
    n_out = int(round(0.01 * x.size))
    pos = g.choice(x.size, size=n_out, replace=False)
    x[pos] *= np.float32(20.0)
    return x.reshape(tiles, 128)


def weight(seed: int = 1, rows: int = 14336, cols: int = 4096, outlier_frac: float = 0.005) -> np.ndarray:
    """bf16 bits, shape (rows, cols)."""
    g = _rng(seed)
    w = g.standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(0.02)
    n_cols = int(round(outlier_frac * cols))
    if n_cols:
        cols_idx = g.choice(cols, size=n_cols, replace=False)
        t = g.standard_t(4, size=(rows, n_cols)).astype(np.float32)
        w[:, cols_idx] = np.float32(0.02 * 5.0) * t
    return bf16_bits(w)


def kv_seed(layer: int, is_v: int) -> int:
    """RHT seed of one (layer, K|V) call: the per-layer +-1 rotation folds into the sign diagonal."""
    return (layer << 1) | int(is_v)


def kv(layer: int, is_v: int, seed: int = 2, heads: int = 8, tokens: int = 32768, dim: int = 128) -> np.ndarray:
    """bf16 bits, shape (heads, tokens, dim), for one (layer, K|V) call."""
    g = _rng(seed * 1_000_003 + layer * 2 + int(is_v))
    x = g.standard_normal((heads, tokens, dim), dtype=np.float32)
    if not is_v:
        ch_rng = _rng(seed * 7919 + layer)
        for h in range(heads):
            ch = ch_rng.choice(dim, size=4, replace=False)
            x[h, :, ch] *= np.float32(10.0)
    return bf16_bits(x)


def model_shapes(layers: int = 32, hidden: int = 4096, inter: int = 14336, q_heads: int = 32,
                 kv_heads: int = 8, head_dim: int = 128):
    """(name, (out_features, in_features)) of every linear weight; tiles run along in_features."""
    shapes = []
    for layer in range(layers):
        shapes += [
            (f"l{layer}.q", (q_heads * head_dim, hidden)),
            (f"l{layer}.k", (kv_heads * head_dim, hidden)),
            (f"l{layer}.v", (kv_heads * head_dim, hidden)),
            (f"l{layer}.o", (hidden, q_heads * head_dim)),
            (f"l{layer}.gate", (inter, hidden)),
            (f"l{layer}.up", (inter, hidden)),
            (f"l{layer}.down", (hidden, inter)),
        ]
    return shapes


def model_tensor(i: int, shape) -> np.ndarray:
    g = _rng(1000 + i)
    w = g.standard_normal(shape, dtype=np.float32)
    w *= np.float32(0.02)
    return bf16_bits(w)


def gaussian(n: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    g = _rng(seed)
    x = g.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def device_normal_bf16(n: int, seed: int, std: float = 0.02, device: str = "cuda"):
    """n bf16 values N(0, std^2) drawn on the GPU with torch's seeded generator (for tensors too
    large to draw on the host in reasonable time); returns the torch tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.empty(n, dtype=torch.bfloat16, device=device)
    step = 1 << 28
    for i in range(0, n, step):
        m = min(step, n - i)
        x[i:i + m] = (torch.randn(m, generator=g, device=device) * std).to(torch.bfloat16)
    return x
