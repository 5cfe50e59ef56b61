"""Seeded synthetic inputs for the sparse-MoE FFN layer forward.

This module is shared by the oracle side and the HIP side.  It holds no part
of the layer's arithmetic: it only draws random tensors of the shapes and
distributions of the five workloads and packs them as float32 or as bfloat16
bit patterns (uint16, round-to-nearest-even from float32).

Workloads (shapes from the models the pages name; distributions as stated):

  tiny      T=64    d=32   h=128   E=4   k=2  S=0  no capacity   fp32, biases 0
  switch    T=4096  d=512  h=2048  E=64  k=1  S=0  cf=1.25       fp32
  mixtral   T=8192  d=4096 h=14336 E=8   k=2  S=0  no capacity   bf16
  glam      T=16384 d=2048 h=8192  E=64  k=2  S=0  cf=1.5        bf16, router bias N(0,1)
  deepseek  T=4096  d=7168 h=2048  E=256 k=8  S=1  no capacity   bf16

x ~ N(0,1); router and expert weights ~ N(0, 0.02); expert biases ~ N(0, 0.02)
(zero for ``tiny``); the ``glam`` router bias ~ N(0,1) in fp32 skews the
expert loads so that the capacity limit drops assignments.  Any workload can
be overridden to the Mixtral expert form (``activation="silu"``,
``expert_bias=False``) or given a ``min_capacity``.

Every tensor is drawn per (tensor id, expert id) from its own PCG64 stream
``SeedSequence(seed, spawn_key=(tensor_id, expert_id))`` so one expert can be
regenerated on its own (the deepseek-shaped weights are 15 GB in bf16).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# tensor ids of the per-(tensor, expert) random streams
TID_X, TID_WG, TID_W1, TID_B1, TID_W2, TID_B2, TID_BG, TID_BSEL = range(8)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    h: int
    E: int
    k: int
    S: int = 0               # shared experts
    cf: float = 0.0          # capacity factor, <= 0 means no limit
    dtype: str = "f32"       # "f32" or "bf16"
    bias_std: float = 0.02   # std of b1, b2 (0 => zero biases)
    w_std: float = 0.02
    router_bias_std: float = 0.0  # std of the fp32 router logit bias (0 => none)
    activation: str = "gelu"      # expert activation, "gelu" or "silu"
    expert_bias: bool = True      # False: bias-free expert Linears (b1, b2 are None)
    min_capacity: int = 0         # floor under the capacity when cf > 0
    sel_bias_std: float = 0.0     # std of the fp32 selection-only router bias (0 => none)

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": MoEConfig("tiny", T=64, d=32, h=128, E=4, k=2, S=0, cf=0.0, dtype="f32", bias_std=0.0),
    "switch": MoEConfig("switch", T=4096, d=512, h=2048, E=64, k=1, S=0, cf=1.25, dtype="f32"),
    "mixtral": MoEConfig("mixtral", T=8192, d=4096, h=14336, E=8, k=2, S=0, cf=0.0, dtype="bf16"),
    "glam": MoEConfig("glam", T=16384, d=2048, h=8192, E=64, k=2, S=0, cf=1.5, dtype="bf16",
                      router_bias_std=1.0),
    "deepseek": MoEConfig("deepseek", T=4096, d=7168, h=2048, E=256, k=8, S=1, cf=0.0, dtype="bf16"),
}


def _rng(seed: int, tid: int, eid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, eid))))


def _normal(seed: int, tid: int, eid: int, shape, std: float) -> np.ndarray:
    a = _rng(seed, tid, eid).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest, ties to even.

    Inputs are finite normal draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def _pack(cfg: MoEConfig, a: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(a) if cfg.dtype == "bf16" else a


class MoEInputs:
    """Lazily generated inputs of one workload.

    Arrays are float32 (``dtype == "f32"``) or uint16 bfloat16 bit patterns
    (``dtype == "bf16"``).  Expert parameters are indexed 0..E-1 for routed
    experts and E..E+S-1 for shared experts.
    """

    def __init__(self, cfg: MoEConfig, seed: int = 0):
        self.cfg = cfg
        self.seed = seed
        self._x = None
        self._wg = None
        self._bg = None
        self._bsel = None

    # token activations [T, d]
    @property
    def x(self) -> np.ndarray:
        if self._x is None:
            c = self.cfg
            self._x = _pack(c, _normal(self.seed, TID_X, 0, (c.T, c.d), 1.0))
        return self._x

    # router weight [E, d] (nn.Linear layout: out x in)
    @property
    def W_g(self) -> np.ndarray:
        if self._wg is None:
            c = self.cfg
            self._wg = _pack(c, _normal(self.seed, TID_WG, 0, (c.E, c.d), c.w_std))
        return self._wg

    # optional fp32 router logit bias [E]
    @property
    def b_g(self) -> Optional[np.ndarray]:
        c = self.cfg
        if c.router_bias_std <= 0:
            return None
        if self._bg is None:
            self._bg = _normal(self.seed, TID_BG, 0, (c.E,), c.router_bias_std)
        return self._bg

    # optional fp32 selection-only router bias [E]
    @property
    def b_sel(self) -> Optional[np.ndarray]:
        c = self.cfg
        if c.sel_bias_std <= 0:
            return None
        if self._bsel is None:
            self._bsel = _normal(self.seed, TID_BSEL, 0, (c.E,), c.sel_bias_std)
        return self._bsel

    def expert(self, e: int):
        """(W1 [h,d], b1 [h], W2 [d,h], b2 [d]) of expert e (routed or shared);
        b1 and b2 are None for bias-free experts."""
        c = self.cfg
        W1 = _pack(c, _normal(self.seed, TID_W1, e, (c.h, c.d), c.w_std))
        W2 = _pack(c, _normal(self.seed, TID_W2, e, (c.d, c.h), c.w_std))
        if not c.expert_bias:
            b1 = b2 = None
        elif c.bias_std > 0:
            b1 = _pack(c, _normal(self.seed, TID_B1, e, (c.h,), c.bias_std))
            b2 = _pack(c, _normal(self.seed, TID_B2, e, (c.d,), c.bias_std))
        else:
            dt = np.uint16 if c.dtype == "bf16" else np.float32
            b1 = np.zeros((c.h,), dtype=dt)
            b2 = np.zeros((c.d,), dtype=dt)
        return W1, b1, W2, b2

    def stacked(self):
        """All expert parameters stacked: W1 [E+S,h,d], b1 [E+S,h], W2 [E+S,d,h],
        b2 [E+S,d] (b1 and b2 None for bias-free experts)."""
        c = self.cfg
        n = c.E + c.S
        dt = np.uint16 if c.dtype == "bf16" else np.float32
        W1 = np.empty((n, c.h, c.d), dtype=dt)
        W2 = np.empty((n, c.d, c.h), dtype=dt)
        b1 = np.empty((n, c.h), dtype=dt) if c.expert_bias else None
        b2 = np.empty((n, c.d), dtype=dt) if c.expert_bias else None

        def fill(e):
            W1[e], eb1, W2[e], eb2 = self.expert(e)
            if c.expert_bias:
                b1[e], b2[e] = eb1, eb2

        # numpy's generators release the GIL, so experts are drawn in parallel
        with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
            list(ex.map(fill, range(n)))
        return W1, b1, W2, b2


def make_inputs(name_or_cfg, seed: int = 0, **overrides) -> MoEInputs:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if overrides:
        cfg = cfg.replace(**overrides)
    return MoEInputs(cfg, seed)
