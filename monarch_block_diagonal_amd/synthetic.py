"""Seeded synthetic inputs for the Monarch workloads.

This module holds no Monarch arithmetic: it draws random numbers, scales them
to the stated variance and rounds them to bfloat16 where a workload is bf16.
The oracle-side tests, the GPU parity tests and the benchmark all take their
inputs from here, so both sides see bit-identical values.

Workloads follow the shapes of the pages' examples: the square Monarch
matrices of Definition C.3 (page 4, "Definition C.3" issue thread), the
GPT-2-small FFN up-projection, the recommender MLP 10000x1024x512 of the
efficiency table (page 4, "efficiency testing numbers" thread) and a large
square layer. Generation: numpy PCG64, seed = 20220401 + 100*cfg + tensor id,
values drawn in fp32, scaled by sqrt(variance), then rounded to nearest-even
bfloat16 for bf16 workloads.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

BASE_SEED = 20220401

# tensor ids used in the seed formula
TID_X, TID_W1, TID_W2, TID_DY = 0, 1, 2, 3
TID_W1_L2, TID_W2_L2 = 11, 12
TID_BIAS = 4


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); returns fp32
    arrays holding exactly representable bf16 values. NaN stays NaN."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    u = a32.view(np.uint32)
    # finite values never wrap: the largest finite pattern 0xFF7FFFFF + 0x8000 fits in 32 bits
    r = u + np.uint32(0x7FFF)
    r += (u >> np.uint32(16)) & np.uint32(1)
    r &= np.uint32(0xFFFF0000)
    nan = np.isnan(a32)
    if nan.any():
        r[nan] = (a32.view(np.uint32)[nan] | np.uint32(0x00400000)) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(a32.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp32 values that are exactly representable in bf16."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    return (a32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Layer:
    in_features: int
    out_features: int
    nblocks1: int
    nblocks2: int
    relu: bool = False            # activation fused after this layer
    mid_features: int = 0         # intermediate width (0: out_features)
    bias: bool = False

    @property
    def mid(self) -> int:
        return self.mid_features or self.out_features

    @property
    def w1_shape(self) -> Tuple[int, int, int]:
        return (self.nblocks1, self.mid // self.nblocks1, -(-self.in_features // self.nblocks1))

    @property
    def w2_shape(self) -> Tuple[int, int, int]:
        return (self.nblocks2, -(-self.out_features // self.nblocks2), self.mid // self.nblocks2)

    @property
    def params(self) -> int:
        a, b, c = self.w1_shape
        d, e, f = self.w2_shape
        return a * b * c + d * e * f


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg: int                      # index used in the seed formula
    layers: Tuple[Layer, ...]
    batch: int
    dtype: str                    # "f32" or "bf16"
    x_dist: str                   # "normal" or "uniform"
    x_var: float                  # variance for normal X
    w_var: Tuple[Tuple[float, float], ...]   # per layer (var R, var L)
    dy_var: float = 1.0
    passes: str = "fwd+bwd"

    @property
    def params(self) -> int:
        return sum(l.params for l in self.layers)


def _recsys(nb: int, batch: int) -> Workload:
    l1 = Layer(10000, 1024, nb, nb, relu=True)
    l2 = Layer(1024, 512, nb, nb, relu=False)
    # variance 1/block_in per stage: 1/q1i for R, 1/q2i for L
    wv = tuple((1.0 / l.w1_shape[2], 1.0 / l.w2_shape[2]) for l in (l1, l2))
    return Workload(f"recsys_mlp_10000x1024x512_nb{nb}_b{batch}", 3, (l1, l2), batch, "f32",
                    "uniform", 1.0, wv)


WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


_add(Workload("tiny_square_n16_b4", 0, (Layer(16, 16, 4, 4),), 8, "f32", "normal", 0.25,
              ((0.25, 0.25),), passes="fwd"))
_add(Workload("square_n1024_b32", 1, (Layer(1024, 1024, 32, 32),), 4096, "bf16", "normal", 1.0,
              ((1.0 / 32, 1.0 / 32),)))
_add(Workload("gpt2_ffn_up_768x3072_nb4", 2, (Layer(768, 3072, 4, 4),), 16 * 1024, "bf16",
              "normal", 1.0, ((1.0 / 192, 1.0 / 192),)))
for _nb in (4, 16):
    for _b in (10, 1000, 10000):
        _add(_recsys(_nb, _b))
# the same FFN up-projection with the MonarchLinear sizes (expanding branch:
# mid = in = 768, stage-1 blocks 4 x (192 x 192), stage-2 blocks 4 x (768 x 192))
# and a bias
_add(Workload("gpt2_ffn_up_monarchlinear_768x3072_nb4_bias", 2,
              (Layer(768, 3072, 4, 4, mid_features=768, bias=True),), 16 * 1024, "bf16",
              "normal", 1.0, ((1.0 / 192, 1.0 / 192),)))
_add(Workload("square_n16384_b128", 4, (Layer(16384, 16384, 128, 128),), 65536, "bf16",
              "normal", 1.0, ((1.0 / 128, 1.0 / 128),)))


def seed_for(cfg: int, tensor_id: int) -> int:
    return BASE_SEED + 100 * cfg + tensor_id


def draw(seed: int, shape, dist: str = "normal", var: float = 1.0, dtype: str = "f32",
         rows: slice | None = None) -> np.ndarray:
    """Draw a seeded fp32 tensor; `rows` optionally keeps only a leading-row slice
    (the full tensor is still drawn so the values match the full draw)."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        a = rng.standard_normal(shape, dtype=np.float32)
        if var != 1.0:
            a *= np.float32(np.sqrt(var))
    elif dist == "uniform":
        a = rng.random(shape, dtype=np.float32)
    else:
        raise ValueError(dist)
    if rows is not None:
        a = np.ascontiguousarray(a[rows])
    if dtype == "bf16":
        a = round_to_bf16(a)
    return a


def make_layer_inputs(w: Workload, layer_index: int = 0, batch: int | None = None,
                      with_dy: bool = True) -> Dict[str, np.ndarray]:
    """Inputs of one layer of a workload: x, w1 (R), w2 (L) and dy (fp32 arrays,
    bf16-exact values for bf16 workloads). Layer 2 of the MLP takes its x from
    layer 1's output, so only its weights are drawn here."""
    layer = w.layers[layer_index]
    b = w.batch if batch is None else batch
    t1, t2 = (TID_W1, TID_W2) if layer_index == 0 else (TID_W1_L2, TID_W2_L2)
    vr, vl = w.w_var[layer_index]
    out = {
        "w1": draw(seed_for(w.cfg, t1), layer.w1_shape, "normal", vr, w.dtype),
        "w2": draw(seed_for(w.cfg, t2), layer.w2_shape, "normal", vl, w.dtype),
    }
    if layer.bias:
        out["bias"] = draw(seed_for(w.cfg, TID_BIAS + 10 * layer_index), (layer.out_features,),
                           "normal", 0.25, w.dtype)
    if layer_index == 0:
        out["x"] = draw(seed_for(w.cfg, TID_X), (b, layer.in_features), w.x_dist, w.x_var, w.dtype)
    if with_dy:
        dy_layer = w.layers[-1]
        out["dy"] = draw(seed_for(w.cfg, TID_DY), (b, dy_layer.out_features), "normal",
                         w.dy_var, w.dtype)
    return out
