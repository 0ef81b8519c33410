"""Seeded generators for K, V and query tensors.

Recipe (the same for every consumer):
- base seed 20260427 + config index; every (tensor, index) pair gets its own
  ``SeedSequence(base, spawn_key=(tensor_id, index))`` so that one layer or one
  decode step can be drawn without drawing the others;
- K, per (layer, KV head): d channel scales ~ LogNormal(0, 0.5); two distinct
  channels chosen uniformly are multiplied by 10; K = fp16(z * scale) with
  z ~ N(0, 1) drawn as float32 in C order over [T][d];
- V: fp16 of float32 N(0, 1), or of Student-t with 4 degrees of freedom (variance 2,
  no rescaling) for the heavy-tailed workload;
- queries for one decode step: float32 N(0, 1) of shape [L][A][H*G][d].
All arrays are C-contiguous numpy arrays.
"""

import numpy as np

from .configs import Config

BASE_SEED = 20260427
_K, _V, _Q, _KSCALE = 0, 1, 2, 3


def _rng(cfg: Config, tensor_id: int, index: int) -> np.random.Generator:
    ss = np.random.SeedSequence(BASE_SEED + cfg.index, spawn_key=(tensor_id, index))
    return np.random.Generator(np.random.PCG64(ss))


def k_channel_scales(cfg: Config, layer: int) -> np.ndarray:
    """float32 [H][d] per-channel scales of one layer, outliers included."""
    rng = _rng(cfg, _KSCALE, layer)
    H, d = cfg.n_kv_heads, cfg.head_dim
    scales = rng.lognormal(0.0, 0.5, size=(H, d)).astype(np.float32)
    for h in range(H):
        ch = rng.choice(d, size=2, replace=False)
        scales[h, ch] *= np.float32(10.0)
    return scales


def gen_k_layer(cfg: Config, layer: int) -> np.ndarray:
    """fp16 [H][T][d] keys of one layer."""
    rng = _rng(cfg, _K, layer)
    H, T, d = cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim
    z = rng.standard_normal((H, T, d), dtype=np.float32)
    z *= k_channel_scales(cfg, layer)[:, None, :]
    return z.astype(np.float16)


def gen_v_layer(cfg: Config, layer: int) -> np.ndarray:
    """fp16 [H][T][d] values of one layer."""
    rng = _rng(cfg, _V, layer)
    shape = (cfg.n_kv_heads, cfg.n_tokens, cfg.head_dim)
    if cfg.v_dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif cfg.v_dist == "student_t4":
        x = rng.standard_t(4.0, size=shape).astype(np.float32)
    else:
        raise ValueError(cfg.v_dist)
    return x.astype(np.float16)


def gen_k(cfg: Config, layers=None) -> np.ndarray:
    """fp16 [L'][H][T][d] keys of the given layers (default: all)."""
    layers = range(cfg.n_layers) if layers is None else layers
    return np.stack([gen_k_layer(cfg, l) for l in layers])


def gen_v(cfg: Config, layers=None) -> np.ndarray:
    layers = range(cfg.n_layers) if layers is None else layers
    return np.stack([gen_v_layer(cfg, l) for l in layers])


def gen_q_step(cfg: Config, step: int) -> np.ndarray:
    """float32 [L][A][H*G][d] queries of one decode step."""
    rng = _rng(cfg, _Q, step)
    shape = (cfg.n_layers, cfg.n_agents, cfg.n_q_heads, cfg.head_dim)
    return rng.standard_normal(shape, dtype=np.float32)
