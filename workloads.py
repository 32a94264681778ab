"""Seeded synthetic inputs for the POET-X orthogonal-equivalence layer.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic. Both the oracle tests and the HIP path take their inputs
from here, so the two sides see bit-identical values.

Citations
  [PX]  page "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
        Transformation" (gist.science, French summary).
  [PX1] page "POET-X：通过扩展正交变换实现内存高效的大语言模型训练"
        (blog.20031104.xyz).

The pages train Llama models on C4 ([PX] Résumé technique §4); no dataset or
trained weight is used here. The layer widths follow a LLaMA-style block at
hidden 2048 ([PX1] 30分钟复现实操路径 names a 1B model with hidden 2048) and
4096, and the block size b=512 appears in [PX] §4 (Llama-3B, b=512).

Recipe, per layer, from one numpy PCG64 stream:
  W0 ~ N(0, 1/n)  [m, n]        (n = fan-in)
  theta_R, theta_P ~ N(0, sigma^2), packed strict upper triangles per block
  pi_R = permutation(m), pi_P = permutation(n)   (int32)
  X  ~ N(0, 1)    [T, n]
  G_Y ~ N(0, 1)   [T, m]        (upstream gradient)
drawn in that order in float64, then cast once (round-to-nearest-even) to the
activation dtype; theta stays float32. Layer streams come from
SeedSequence(1000 * config_id).spawn(number_of_layers), in layer order.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    m: int                      # output features (rows of W0)
    n: int                      # input features (columns of W0)
    bsz_R: tuple                # block sizes of R, summing to m
    bsz_P: tuple                # block sizes of P, summing to n


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    layers: tuple
    k: int                      # Neumann order: powers S^0..S^k
    T: int                      # tokens
    dtype: str                  # "f32" or "bf16" (activations and W0)
    theta_std: float
    backward: bool

    @property
    def seed(self) -> int:
        return 1000 * self.cid


def _uniform(dim: int, b: int) -> tuple:
    assert dim % b == 0
    return (b,) * (dim // b)


def _llama_block(h: int, ff: int, b: int, ff_blocks: tuple) -> tuple:
    sq = _uniform(h, b)
    return (
        LayerSpec("q", h, h, sq, sq),
        LayerSpec("k", h, h, sq, sq),
        LayerSpec("v", h, h, sq, sq),
        LayerSpec("o", h, h, sq, sq),
        LayerSpec("gate", ff, h, ff_blocks, sq),
        LayerSpec("up", ff, h, ff_blocks, sq),
        LayerSpec("down", h, ff, sq, ff_blocks),
    )


WORKLOADS = {
    1: Workload(1, "poetx-layer-256x256-f32", (LayerSpec("layer", 256, 256, _uniform(256, 32), _uniform(256, 32)),),
                k=3, T=64, dtype="f32", theta_std=0.01, backward=True),
    2: Workload(2, "poetx-attn-proj-2048x2048-bf16-fwd", (LayerSpec("attn", 2048, 2048, _uniform(2048, 256), _uniform(2048, 256)),),
                k=4, T=4096, dtype="bf16", theta_std=0.01, backward=False),
    3: Workload(3, "poetx-mlp-up-5632x2048-bf16", (LayerSpec("up", 5632, 2048, _uniform(5632, 256), _uniform(2048, 256)),),
                k=4, T=8192, dtype="bf16", theta_std=0.01, backward=True),
    4: Workload(4, "poetx-llama-block-h2048-7-linears-bf16",
                _llama_block(2048, 5632, 256, _uniform(5632, 256)),
                k=4, T=16384, dtype="bf16", theta_std=0.01, backward=True),
    5: Workload(5, "poetx-llama-block-h4096-7-linears-bf16",
                _llama_block(4096, 11008, 512, (512,) * 21 + (256,)),
                k=5, T=16384, dtype="bf16", theta_std=0.005, backward=True),
}


def n_params(bsz) -> int:
    return sum(b * (b - 1) // 2 for b in bsz)


@dataclasses.dataclass
class LayerInputs:
    spec: LayerSpec
    W0: np.ndarray          # [m, n] float32 values (exactly representable in dtype)
    theta_R: np.ndarray     # float32
    theta_P: np.ndarray     # float32
    pi_R: np.ndarray        # int32 [m]
    pi_P: np.ndarray        # int32 [n]
    X: np.ndarray           # [T, n] float32 values
    G_Y: Optional[np.ndarray]


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws once to the activation dtype; return them as float32."""
    if dtype == "f32":
        return a.astype(np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.bfloat16)
    return t.to(torch.float32).numpy()


def layer_inputs(w: Workload, layer: int, T: Optional[int] = None,
                 draw_grad: bool = True, theta_scale: float = 1.0) -> LayerInputs:
    """Draw one layer's inputs. `T` may shrink the token count for small cases
    (the first rows of a shorter draw differ from the full draw's rows)."""
    spec = w.layers[layer]
    T = w.T if T is None else T
    ss = np.random.SeedSequence(w.seed).spawn(len(w.layers))[layer]
    rng = np.random.default_rng(ss)
    m, n = spec.m, spec.n
    W0 = _cast(rng.standard_normal((m, n)) / np.sqrt(n), w.dtype)
    th_R = (rng.standard_normal(n_params(spec.bsz_R)) * w.theta_std * theta_scale).astype(np.float32)
    th_P = (rng.standard_normal(n_params(spec.bsz_P)) * w.theta_std * theta_scale).astype(np.float32)
    pi_R = rng.permutation(m).astype(np.int32)
    pi_P = rng.permutation(n).astype(np.int32)
    X = _cast(rng.standard_normal((T, n)), w.dtype)
    G = _cast(rng.standard_normal((T, m)), w.dtype) if draw_grad else None
    return LayerInputs(spec, W0, th_R, th_P, pi_R, pi_P, X, G)


def small_case(m: int, n: int, bsz_R, bsz_P, T: int, seed: int, dtype: str = "f32",
               theta_std: float = 0.05) -> LayerInputs:
    """A free-form small layer for edge-case tests (ragged blocks, tiny T)."""
    rng = np.random.default_rng(seed)
    spec = LayerSpec("case", m, n, tuple(bsz_R), tuple(bsz_P))
    W0 = _cast(rng.standard_normal((m, n)) / np.sqrt(n), dtype)
    th_R = (rng.standard_normal(n_params(bsz_R)) * theta_std).astype(np.float32)
    th_P = (rng.standard_normal(n_params(bsz_P)) * theta_std).astype(np.float32)
    pi_R = rng.permutation(m).astype(np.int32)
    pi_P = rng.permutation(n).astype(np.int32)
    X = _cast(rng.standard_normal((T, n)), dtype)
    G = _cast(rng.standard_normal((T, m)), dtype)
    return LayerInputs(spec, W0, th_R, th_P, pi_R, pi_P, X, G)


def workload_layers(w: Workload, T: Optional[int] = None) -> List[LayerInputs]:
    return [layer_inputs(w, i, T=T, draw_grad=w.backward) for i in range(len(w.layers))]
