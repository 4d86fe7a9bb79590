"""Seeded synthetic inputs shared by the HIP path's tests, the bench and the oracle.

This module holds no arithmetic of the method: it draws numbers and, for the
bf16 workloads, rounds them once to bf16-representable float32 values so that
both sides start from identical inputs.

Streams: numpy PCG64 seeded through SeedSequence([seed, group, index]).  Every
weight tensor has its own stream (group = layer), so any single layer can be
regenerated on its own.

Value recipe (the workload definition; the pages fix no initialisation):
  x, target      ~ N(0, 1)
  weight matrices ~ N(0, 0.02^2)
  biases 0, LayerNorm gamma 1, beta 0
"""
from __future__ import annotations

import numpy as np

# Order of the per-layer tensors in the flat parameter vector.  The weight
# matrices are stored [out_features, in_features], row-major.
PARAM_NAMES = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
               "ln2_g", "ln2_b", "w_1", "b_1", "w_2", "b_2")

_MATRIX_ID = {"w_qkv": 0, "w_o": 1, "w_1": 2, "w_2": 3}
_GROUP_DATA = 1 << 20          # stream group for x / target (never a layer index)
WEIGHT_STD = 0.02


def param_shapes(d_model: int, d_ff: int) -> dict:
    d, f = d_model, d_ff
    return {"ln1_g": (d,), "ln1_b": (d,), "w_qkv": (3 * d, d), "b_qkv": (3 * d,),
            "w_o": (d, d), "b_o": (d,), "ln2_g": (d,), "ln2_b": (d,),
            "w_1": (f, d), "b_1": (f,), "w_2": (d, f), "b_2": (d,)}


def _rng(seed: int, group: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, group, index])))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 storage of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def normal(seed: int, group: int, index: int, shape, std: float = 1.0,
           bf16: bool = False) -> np.ndarray:
    v = _rng(seed, group, index).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return round_to_bf16(v) if bf16 else v


def layer_params(seed: int, layer: int, d_model: int, d_ff: int,
                 bf16: bool = False) -> dict:
    """One layer's tensors as float32 arrays (bf16-representable if bf16)."""
    out = {}
    for name, shape in param_shapes(d_model, d_ff).items():
        if name in _MATRIX_ID:
            out[name] = normal(seed, layer, _MATRIX_ID[name], shape, WEIGHT_STD, bf16)
        elif name.endswith("_g"):
            out[name] = np.ones(shape, np.float32)
        else:
            out[name] = np.zeros(shape, np.float32)
    return out


def cell_params(cfg, bf16: bool | None = None) -> list:
    bf = (cfg.precision == "bf16") if bf16 is None else bf16
    return [layer_params(cfg.seed, l, cfg.d_model, cfg.d_ff, bf) for l in range(cfg.layers)]


def cell_data(cfg, bf16: bool | None = None, batch: int | None = None):
    """x and target, each [N, S, D] float32 (bf16-representable if bf16)."""
    bf = (cfg.precision == "bf16") if bf16 is None else bf16
    n = cfg.batch if batch is None else batch
    shape = (n, cfg.seq, cfg.d_model)
    return (normal(cfg.seed, _GROUP_DATA, 0, shape, 1.0, bf),
            normal(cfg.seed, _GROUP_DATA, 1, shape, 1.0, bf))


def sequence_data(cfg, index: int, bf16: bool | None = None):
    """x and target of one sequence of the full mini-batch (same values as cell_data)."""
    x, t = cell_data(cfg, bf16)
    return x[index], t[index]


def flatten_params(layers: list, order=PARAM_NAMES) -> np.ndarray:
    """Concatenate per-layer tensors in the flat order (layer-major)."""
    return np.concatenate([np.asarray(p[n], np.float32).ravel() for p in layers for n in order])


def unflatten_params(flat: np.ndarray, n_layers: int, d_model: int, d_ff: int) -> list:
    shapes = param_shapes(d_model, d_ff)
    out, off = [], 0
    for _ in range(n_layers):
        d = {}
        for n in PARAM_NAMES:
            cnt = int(np.prod(shapes[n]))
            d[n] = flat[off:off + cnt].reshape(shapes[n])
            off += cnt
        out.append(d)
    assert off == flat.size, (off, flat.size)
    return out


# ---------------------------------------------------------------- convolutional cell
CONV_NAMES = ("w1", "bn1_g", "bn1_b", "w2", "bn2_g", "bn2_b")
_CONV_MATRIX_ID = {"w1": 10, "w2": 11}


def conv_param_shapes(channels: int) -> dict:
    c = channels
    return {"w1": (c, 3, 3, c), "bn1_g": (c,), "bn1_b": (c,),
            "w2": (c, 3, 3, c), "bn2_g": (c,), "bn2_b": (c,)}


def conv_block_params(seed: int, block: int, channels: int, bf16: bool = False) -> dict:
    """He-normal conv weights (std sqrt(2 / (9 C))), BN gamma 1, beta 0."""
    std = float(np.sqrt(2.0 / (9 * channels)))
    out = {}
    for name, shape in conv_param_shapes(channels).items():
        if name in _CONV_MATRIX_ID:
            out[name] = normal(seed, block, _CONV_MATRIX_ID[name], shape, std, bf16)
        elif name.endswith("_g"):
            out[name] = np.ones(shape, np.float32)
        else:
            out[name] = np.zeros(shape, np.float32)
    return out


def conv_cell_params(cfg, bf16: bool | None = None) -> list:
    bf = (cfg.precision == "bf16") if bf16 is None else bf16
    return [conv_block_params(cfg.seed, l, cfg.channels, bf) for l in range(cfg.blocks)]


def conv_cell_data(cfg, bf16: bool | None = None, batch: int | None = None):
    """x and target [N, H, W, C] (NHWC), ~N(0, 1)."""
    bf = (cfg.precision == "bf16") if bf16 is None else bf16
    n = cfg.batch if batch is None else batch
    shape = (n, cfg.height, cfg.width, cfg.channels)
    return (normal(cfg.seed, _GROUP_DATA, 2, shape, 1.0, bf),
            normal(cfg.seed, _GROUP_DATA, 3, shape, 1.0, bf))
