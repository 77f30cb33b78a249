"""Seeded synthetic layers for the AWQ per-layer search.

This module only draws inputs: weight matrices, calibration activations with a
few outlier channels, and the candidate grids. It holds none of the method's
arithmetic, so both the HIP path and the CPU oracle can be fed from it.

Workloads follow the shapes the AWQ pages discuss: Llama-class projections,
~1 % salient input channels whose activations are much larger than the rest
("AWQ and Activation-Aware Scaling", section "The observation"; the AWQ
reading note, "Key takeaways"), a calibration set of a few hundred sequences
and a grid of about twenty exponents ("05 — AWQ: Activation-Aware Weight
Scaling", section 4). No dataset or trained weights are used: the values are
Gaussian with the stated spreads.

Every array is drawn from numpy's PCG64 keyed by
``SeedSequence([seed, config_id, stream])`` with the streams
0 = W, 1 = X base, 2 = outlier channel indices, 3 = outlier factors, 4 = signs,
10 + l = layer l of a group sharing X, 20 / 21 = a normalisation's weight / bias.
bf16 tensors are produced from float32 draws by one round-to-nearest-even
conversion and are carried as ``uint16`` bit patterns (numpy has no bf16).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DEFAULT_SEED = 2026


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One synthetic linear layer ``Y = X · Wᵀ`` plus the search it gets."""
    name: str
    cid: int                 # config id, part of the seed
    T: int                   # calibration tokens
    N: int                   # output channels (rows of W)
    K: int                   # input channels
    dtype: str               # "bf16", "f16" or "f32" for both X and W
    w_std: float
    n_outliers: int
    out_lo: float
    out_hi: float
    x_kind: str = "normal"   # "normal" or "abs_sign" (|N(0,1)|·sign)
    bits: int = 4
    zero_point: bool = True
    variants: tuple = (True,)  # zero_point settings searched (c5 runs both)
    n_alpha: int = 20
    n_ratio: int = 0         # 0 = no clip search
    pack: bool = False
    group: int = 128
    layers: tuple = ()       # output channels of each linear reading the same X (a group)


CONFIGS = {
    # Single 512x512 fp32 layer, 256 tokens, 5 outlier channels: the small case.
    "layer512_f32": LayerConfig("layer512_f32", 1, 256, 512, 512, "f32", 0.02, 5, 20.0, 100.0),
    # Llama-7B attention projection, 64K calibration tokens (128 x 512).
    "llama7b_attn_4096": LayerConfig("llama7b_attn_4096", 2, 65536, 4096, 4096, "bf16", 0.02, 41,
                                     20.0, 100.0, pack=True),
    # Llama-7B MLP up projection with the clip search.
    "llama7b_mlp_up": LayerConfig("llama7b_mlp_up", 3, 65536, 11008, 4096, "bf16", 0.02, 41,
                                  20.0, 100.0, n_ratio=20, pack=True),
    # Llama-7B MLP down projection, heavy-tailed post-activation inputs, INT3,
    # packed 3-bit.
    "llama7b_mlp_down_int3": LayerConfig("llama7b_mlp_down_int3", 4, 65536, 4096, 11008, "bf16",
                                         0.02, 110, 10.0, 200.0, x_kind="abs_sign", bits=3,
                                         n_ratio=20, pack=True),
    # The attention projection layer at group sizes 32 and 64 (same X and W
    # as llama7b_attn_4096): the group-size comparison.
    "llama7b_attn_4096_g64": LayerConfig("llama7b_attn_4096_g64", 2, 65536, 4096, 4096, "bf16",
                                         0.02, 41, 20.0, 100.0, pack=True, group=64),
    "llama7b_attn_4096_g32": LayerConfig("llama7b_attn_4096_g32", 2, 65536, 4096, 4096, "bf16",
                                         0.02, 41, 20.0, 100.0, pack=True, group=32),
    # The same attention projection held in fp16 (an fp16 model); the same
    # underlying values as llama7b_attn_4096 (config id 2), stored as fp16.
    "llama7b_attn_4096_f16": LayerConfig("llama7b_attn_4096_f16", 2, 65536, 4096, 4096, "f16",
                                         0.02, 41, 20.0, 100.0, pack=True),
    # 70B-class MLP layer, asymmetric and symmetric INT4.
    "llama70b_mlp": LayerConfig("llama70b_mlp", 5, 32768, 28672, 8192, "bf16", 0.015, 82,
                                20.0, 100.0, variants=(True, False), n_ratio=20, pack=True),
    # Llama-7B query/key/value projections: three 4096x4096 linears on the
    # same normalised input, searched with one shared s, which is then folded
    # into the RMSNorm weight; each layer is packed.
    "llama7b_qkv_group": LayerConfig("llama7b_qkv_group", 6, 65536, 12288, 4096, "bf16", 0.02, 41,
                                     20.0, 100.0, pack=True, layers=(4096, 4096, 4096)),
}

BENCH_CONFIG = "llama7b_attn_4096"


def alpha_grid(n: int = 20) -> np.ndarray:
    """``n`` exponents spread evenly over [0, 1], both ends included."""
    return (np.arange(n, dtype=np.float64) / (n - 1)).astype(np.float32)


def ratio_grid(n: int = 20) -> np.ndarray:
    """``n`` clip ratios spread evenly over [0.5, 1.0], both ends included."""
    return (0.5 + np.arange(n, dtype=np.float64) * (0.5 / (n - 1))).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, cid: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, stream])))


def _encode(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values stored as bf16 bits (RNE), fp16 bits (numpy's RNE) or float32."""
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f16":
        return np.ascontiguousarray(a32, dtype=np.float32).astype(np.float16).view(np.uint16)
    return np.ascontiguousarray(a32, dtype=np.float32)


def make_weight(N: int, K: int, w_std: float, dtype: str, seed: int = DEFAULT_SEED,
                cid: int = 0, stream: int = 0) -> np.ndarray:
    """W [N, K] ~ N(0, w_std²), row-major (the out x in layout of a linear layer)."""
    w = _rng(seed, cid, stream).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(w_std)
    return _encode(w, dtype)


def outlier_channels(K: int, n_out: int, lo: float, hi: float, seed: int = DEFAULT_SEED,
                     cid: int = 0):
    """Indices (sorted) and log-uniform [lo, hi] factors of the salient input channels."""
    if n_out == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.float32)
    idx = np.sort(_rng(seed, cid, 2).choice(K, size=n_out, replace=False))
    u = _rng(seed, cid, 3).uniform(np.log(lo), np.log(hi), size=n_out)
    return idx.astype(np.int64), np.exp(u).astype(np.float32)


def make_activations(T: int, K: int, n_out: int, lo: float, hi: float, dtype: str,
                     x_kind: str = "normal", seed: int = DEFAULT_SEED, cid: int = 0,
                     chunk: int = 8192) -> np.ndarray:
    """X [T, K]: N(0,1) (or |N(0,1)|·sign) with ``n_out`` channels scaled up.

    Drawn in token chunks so a 65536 x 11008 layer never holds a float64 copy.
    The outlier factor is applied in float32 before the single rounding to
    the stored type (bf16 or fp16 bits, or float32).
    """
    idx, fac = outlier_channels(K, n_out, lo, hi, seed, cid)
    g = _rng(seed, cid, 1)
    gs = _rng(seed, cid, 4) if x_kind == "abs_sign" else None
    out = np.empty((T, K), dtype=np.uint16 if dtype in ("bf16", "f16") else np.float32)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        x = g.standard_normal((t1 - t0, K), dtype=np.float32)
        if gs is not None:
            sgn = np.where(gs.standard_normal((t1 - t0, K), dtype=np.float32) < 0,
                           np.float32(-1), np.float32(1))
            x = np.abs(x) * sgn
        if n_out:
            x[:, idx] *= fac[None, :]
        out[t0:t1] = _encode(x, dtype)
    return out


def make_layer(cfg: LayerConfig, seed: int = DEFAULT_SEED, T: Optional[int] = None):
    """(X, W) for a config; ``T`` may shorten the calibration set (same first rows)."""
    T = cfg.T if T is None else T
    X = make_activations(T, cfg.K, cfg.n_outliers, cfg.out_lo, cfg.out_hi, cfg.dtype,
                         cfg.x_kind, seed, cfg.cid)
    W = make_weight(cfg.N, cfg.K, cfg.w_std, cfg.dtype, seed, cfg.cid)
    return X, W


def make_group(cfg: LayerConfig, seed: int = DEFAULT_SEED, T: Optional[int] = None):
    """(X, [W_l]) for a config whose linears share X; layer l's weights come
    from stream 10 + l."""
    T = cfg.T if T is None else T
    X = make_activations(T, cfg.K, cfg.n_outliers, cfg.out_lo, cfg.out_hi, cfg.dtype,
                         cfg.x_kind, seed, cfg.cid)
    Ws = [make_weight(n, cfg.K, cfg.w_std, cfg.dtype, seed, cfg.cid, 10 + l)
          for l, n in enumerate(cfg.layers)]
    return X, Ws


def make_norm_weight(K: int, dtype: str, seed: int = DEFAULT_SEED, cid: int = 0,
                     with_bias: bool = False):
    """Per-channel weight γ ~ 1 + 0.1·N(0,1) (and bias β ~ 0.05·N(0,1)) of a
    normalisation, from streams 20 and 21."""
    g = (1.0 + 0.1 * _rng(seed, cid, 20).standard_normal(K)).astype(np.float32)
    b = (0.05 * _rng(seed, cid, 21).standard_normal(K)).astype(np.float32) if with_bias else None
    return _encode_any(g, dtype), None if b is None else _encode_any(b, dtype)


def _encode_any(a32: np.ndarray, dtype: str) -> np.ndarray:
    return _encode(a32, dtype)


def make_custom(T: int, N: int, K: int, dtype: str = "bf16", n_out: Optional[int] = None,
                w_std: float = 0.02, lo: float = 20.0, hi: float = 100.0,
                x_kind: str = "normal", seed: int = DEFAULT_SEED, cid: int = 100):
    """A layer of any shape with ~1 % outlier channels (at least one when K >= 32)."""
    if n_out is None:
        n_out = max(1, K // 100) if K >= 32 else 0
    X = make_activations(T, K, n_out, lo, hi, dtype, x_kind, seed, cid)
    W = make_weight(N, K, w_std, dtype, seed, cid)
    return X, W
