"""Seeded synthetic inputs for the ST-DiT attention-block workloads.

This module is shared by the fp64 oracle and the HIP path and therefore holds
none of the block's arithmetic: only the workload shape table, random draws,
and the rounding of those draws to bf16 storage (round-to-nearest-even).

Workloads stand in for the video and image DiT shapes the pages describe
(ScaleFusion review, "Experimental results": OpenSora v1.2 ST-DiT at 1080p;
xDiT, "Experiments": image DiTs up to 4096px).  No dataset or trained weight is
used: activations are N(0, 1) and weights N(0, 0.02^2), drawn from numpy's
PCG64 with a per-workload SeedSequence.

Weight layout is "out-features major" (the layout of a linear layer's weight):
  w_qkv : [3*H*d, C]   rows 0..H*d-1 produce q, then k, then v
  w_o   : [C, H*d]
"""
from __future__ import annotations

import numpy as np

# Workload table.  grid_w is the width of the latent patch grid; S = grid_w * grid_h.
CONFIGS = {
    1: dict(name="tiny_fp32", B=1, T=4, S=64, grid_w=8, C=128, H=2, d=64, dtype="f32"),
    2: dict(name="720p_4s", B=1, T=24, S=3600, grid_w=80, C=1152, H=16, d=72, dtype="bf16"),
    3: dict(name="1080p_8s", B=1, T=51, S=8160, grid_w=120, C=1152, H=16, d=72, dtype="bf16"),
    # 1080p under the slicing schedule: T padded 51 -> 52 with a zero frame.
    4: dict(name="1080p_8s_sliced", B=1, T=52, t_valid=51, S=8160, grid_w=120, C=1152, H=16,
            d=72, dtype="bf16", n_t=4, n_s=4),
    5: dict(name="image_4096px", B=1, T=1, S=65536, grid_w=256, C=384, H=3, d=128, dtype="bf16"),
}

EPS = 1e-6
ROPE_BASE = 10000.0
W_STD = 0.02


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest-even; returns the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, chunk: int = 1 << 24) -> np.ndarray:
    """float32 N(0, std^2), drawn in chunks so huge tensors do not need a float64 copy."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        rng.standard_normal(e - s, dtype=np.float32, out=out[s:e])
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def _storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32


def make_inputs(cfg_id: int, *, with_x: bool = True) -> dict:
    """Inputs of one workload, in storage form (uint16 bf16 bits, or float32 for "f32").

    Streams: SeedSequence(1000 + base_cfg).spawn(5) -> x, w_qkv spatial, w_o spatial,
    w_qkv temporal, w_o temporal.  Workload 4 reuses workload 3's draws and appends a
    zero frame at t = 51.
    """
    cfg = dict(CONFIGS[cfg_id])
    base_id = 3 if cfg_id == 4 else cfg_id
    base = CONFIGS[base_id]
    B, T, S, C, H, d, dt = base["B"], base["T"], base["S"], base["C"], base["H"], base["d"], base["dtype"]
    ss = np.random.SeedSequence(1000 + base_id).spawn(5)
    rngs = [np.random.Generator(np.random.PCG64(s)) for s in ss]
    hd = H * d
    out = dict(cfg=cfg, cfg_id=cfg_id)
    if with_x:
        x = _storage(_normal(rngs[0], (B, T, S, C), 1.0), dt)
        if cfg_id == 4:
            pad = np.zeros((B, cfg["T"] - T, S, C), dtype=x.dtype)
            x = np.concatenate([x, pad], axis=1)
        out["x"] = x
    out["w_qkv_s"] = _storage(_normal(rngs[1], (3 * hd, C), W_STD), dt)
    out["w_o_s"] = _storage(_normal(rngs[2], (C, hd), W_STD), dt)
    out["w_qkv_t"] = _storage(_normal(rngs[3], (3 * hd, C), W_STD), dt)
    out["w_o_t"] = _storage(_normal(rngs[4], (C, hd), W_STD), dt)
    out["g_q"] = np.ones(d, dtype=np.float32)
    out["g_k"] = np.ones(d, dtype=np.float32)
    return out


def randn(shape, seed: int, std: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """Generic seeded N(0, std^2) tensor in storage form, for tests at arbitrary shapes."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return _storage(_normal(rng, tuple(shape), std), dtype)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Storage form (bf16 bits or float32) widened exactly to float64."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def bits(shape, seed: int, dtype: str = "bf16") -> np.ndarray:
    """Uniformly random storage words (uint16 for bf16, uint32 reinterpreted as float32 for f32), seeded.

    For pure data movement (relayouts, exchanges): every bit pattern is as good as any other, and
    distinct words make a misplaced element visible.  Float32 words avoid the NaN range."""
    r = np.random.default_rng(seed)
    if dtype == "bf16":
        return r.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    return r.integers(0, 0x7F000000, size=shape, dtype=np.uint32).view(np.float32)

