"""Seeded synthetic inputs for the MoE layer: activations, router, experts.

This module is shared by the tests, the benchmark and the oracle's callers. It holds
no arithmetic of the layer itself: it only draws numbers and stores them.

Recipe (every tensor has its own numpy PCG64 stream ``default_rng([seed, tag, index])``
so that experts can be produced one at a time and regenerated on demand):

* draws are float32 N(0, 1) scaled by the tensor's std, then (bf16 workloads) rounded
  to bfloat16 with round-to-nearest-even and kept as uint16 bit patterns;
* x ~ N(0, 1); router, gate and up weights std 1/sqrt(d); down weights std 1/sqrt(f)
  (std = 1/sqrt(fan_in));
* router bias: none; "zipf" = a seeded permutation gives each expert a rank r in 1..E,
  w = r^-s, and the bias is w min-max scaled linearly onto [-2, 2]; "normal" = N(0, std).
* output gradient of the backward pass: dy ~ N(0, 1) [T][d], stored like x;
* FP8 expert weights (weights == "fp8_e4m3"): the same float32 draws, quantised per output
  row: scale = max |row| / 448 (the largest E4M3 value), codes = torch's float8_e4m3fn
  cast (round to nearest) of row / scale. This is how a checkpoint would be converted; the
  library and the oracle only ever see the codes and the scales.

Memory layout of every weight is out-features-major (the layout of a linear layer's
weight): router [E][d], gate and up [E][f][d], down [E][d][f], shared gate/up
[n_s][f_s][d], shared down [n_s][d][f_s]. The matrix products are the ones of the
row-vector convention y = x . W with W = stored^T.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

from .configs import LayerConfig

TAG_X, TAG_WR, TAG_BIAS, TAG_WG, TAG_WU, TAG_WD, TAG_SWG, TAG_SWU, TAG_SWD, TAG_PERM, TAG_DY = range(11)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).copy()
    b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 values they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


E4M3_MAX = 448.0


def quantize_rows_e4m3(a: np.ndarray):
    """float32 [rows, cols] -> (E4M3 codes uint8 [rows, cols], float32 scale [rows]): one
    scale per row, max |row| / 448 (1 for an all-zero row), codes = round-to-nearest cast of
    row / scale (clamped to +-448 first, so no code is NaN)."""
    import torch
    a = np.ascontiguousarray(a, dtype=np.float32)
    amax = np.abs(a).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = torch.from_numpy(a / scale[:, None]).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), scale


def _normal(seed: int, tag: int, index: int, shape, std: float) -> np.ndarray:
    a = np.random.default_rng([seed, tag, index]).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


@dataclass
class LayerInputs:
    """Host-side inputs of one layer. ``storage`` arrays are what is uploaded
    (uint16 bf16 bits or float32); ``values(...)`` gives their exact float32 values."""
    cfg: LayerConfig
    x: np.ndarray  # [T, d] storage
    w_router: np.ndarray  # [E, d] storage
    router_bias: Optional[np.ndarray]  # [E] float32 or None

    def _store(self, a32: np.ndarray) -> np.ndarray:
        return to_bf16_bits(a32) if self.cfg.dtype == "bf16" else a32

    def values(self, storage: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(storage) if self.cfg.dtype == "bf16" else storage

    # ---- routed experts ------------------------------------------------
    def expert(self, e: int):
        c = self.cfg
        sd, sf = 1.0 / math.sqrt(c.d_model), 1.0 / math.sqrt(c.d_ff)
        wg = self._store(_normal(c.seed, TAG_WG, e, (c.d_ff, c.d_model), sd))
        wu = self._store(_normal(c.seed, TAG_WU, e, (c.d_ff, c.d_model), sd))
        wd = self._store(_normal(c.seed, TAG_WD, e, (c.d_model, c.d_ff), sf))
        return wg, wu, wd

    def expert_values(self, e: int):
        if self.cfg.fp8:
            raise ValueError("FP8 expert weights are codes and scales: decode them with the oracle")
        return tuple(self.values(w) for w in self.expert(e))

    def expert_fp8(self, e: int):
        """FP8 routed expert e: (gate codes [f][d], up codes [f][d], down codes [d][f],
        gate scale [f], up scale [f], down scale [d])."""
        c = self.cfg
        sd, sf = 1.0 / math.sqrt(c.d_model), 1.0 / math.sqrt(c.d_ff)
        cg, sg = quantize_rows_e4m3(_normal(c.seed, TAG_WG, e, (c.d_ff, c.d_model), sd))
        cu, su = quantize_rows_e4m3(_normal(c.seed, TAG_WU, e, (c.d_ff, c.d_model), sd))
        cdn, sdn = quantize_rows_e4m3(_normal(c.seed, TAG_WD, e, (c.d_model, c.d_ff), sf))
        return cg, cu, cdn, sg, su, sdn

    # ---- shared experts ------------------------------------------------
    def shared(self, s: int):
        c = self.cfg
        sd, sf = 1.0 / math.sqrt(c.d_model), 1.0 / math.sqrt(c.d_ff_shared)
        wg = self._store(_normal(c.seed, TAG_SWG, s, (c.d_ff_shared, c.d_model), sd))
        wu = self._store(_normal(c.seed, TAG_SWU, s, (c.d_ff_shared, c.d_model), sd))
        wd = self._store(_normal(c.seed, TAG_SWD, s, (c.d_model, c.d_ff_shared), sf))
        return wg, wu, wd

    def shared_values(self, s: int):
        if self.cfg.fp8:
            raise ValueError("FP8 expert weights are codes and scales: decode them with the oracle")
        return tuple(self.values(w) for w in self.shared(s))

    def shared_fp8(self, s: int):
        """FP8 shared expert s, in the order of expert_fp8."""
        c = self.cfg
        sd, sf = 1.0 / math.sqrt(c.d_model), 1.0 / math.sqrt(c.d_ff_shared)
        cg, sg = quantize_rows_e4m3(_normal(c.seed, TAG_SWG, s, (c.d_ff_shared, c.d_model), sd))
        cu, su = quantize_rows_e4m3(_normal(c.seed, TAG_SWU, s, (c.d_ff_shared, c.d_model), sd))
        cdn, sdn = quantize_rows_e4m3(_normal(c.seed, TAG_SWD, s, (c.d_model, c.d_ff_shared), sf))
        return cg, cu, cdn, sg, su, sdn

    # ---- bulk production ---------------------------------------------
    def for_each_expert(self, fn: Callable[[int, tuple], None], threads: int = 8,
                        shared: bool = False) -> None:
        """Call fn(index, (wg, wu, wd)) for every routed (or shared) expert, producing
        them on ``threads`` threads (numpy releases the GIL while drawing). FP8 layers pass
        the six arrays of expert_fp8 instead."""
        n = self.cfg.n_shared if shared else self.cfg.n_experts
        if self.cfg.fp8:
            make = self.shared_fp8 if shared else self.expert_fp8
        else:
            make = self.shared if shared else self.expert

        def work(i):
            fn(i, make(i))

        if threads <= 1 or n <= 1:
            for i in range(n):
                work(i)
            return
        with ThreadPoolExecutor(max_workers=min(threads, n)) as ex:
            list(ex.map(work, range(n)))

    def stacked_experts(self, threads: int = 8):
        """All routed experts as three stacked storage arrays [E,f,d], [E,f,d], [E,d,f]."""
        c = self.cfg
        dt = np.uint16 if c.dtype == "bf16" else np.float32
        wg = np.empty((c.n_experts, c.d_ff, c.d_model), dt)
        wu = np.empty_like(wg)
        wd = np.empty((c.n_experts, c.d_model, c.d_ff), dt)

        def put(e, w):
            wg[e], wu[e], wd[e] = w

        self.for_each_expert(put, threads)
        return wg, wu, wd

    def stacked_shared(self):
        c = self.cfg
        if c.n_shared == 0:
            return None
        dt = np.uint16 if c.dtype == "bf16" else np.float32
        wg = np.empty((c.n_shared, c.d_ff_shared, c.d_model), dt)
        wu = np.empty_like(wg)
        wd = np.empty((c.n_shared, c.d_model, c.d_ff_shared), dt)
        for s in range(c.n_shared):
            wg[s], wu[s], wd[s] = self.shared(s)
        return wg, wu, wd


def router_bias_values(cfg: LayerConfig) -> Optional[np.ndarray]:
    E = cfg.n_experts
    if cfg.router_bias == "none":
        return None
    if cfg.router_bias == "zipf":
        rank = np.random.default_rng([cfg.seed, TAG_PERM, 0]).permutation(E).astype(np.float64) + 1.0
        w = rank ** (-cfg.bias_scale)
        return (4.0 * (w - w.min()) / (w.max() - w.min()) - 2.0).astype(np.float32)
    if cfg.router_bias == "normal":
        return _normal(cfg.seed, TAG_BIAS, 0, (E,), cfg.bias_scale)
    raise ValueError(f"unknown router bias recipe {cfg.router_bias!r}")


def output_grad(cfg: LayerConfig) -> np.ndarray:
    """dy [T][d] for the backward pass (storage format of x)."""
    a = _normal(cfg.seed, TAG_DY, cfg.x_stream, (cfg.T, cfg.d_model), 1.0)
    return to_bf16_bits(a) if cfg.dtype == "bf16" else a


def make_inputs(cfg: LayerConfig) -> LayerInputs:
    """Activations, router weight and bias of ``cfg`` (experts are produced on demand)."""
    store = to_bf16_bits if cfg.dtype == "bf16" else (lambda a: a)
    x = store(_normal(cfg.seed, TAG_X, cfg.x_stream, (cfg.T, cfg.d_model), 1.0))
    wr = store(_normal(cfg.seed, TAG_WR, 0, (cfg.n_experts, cfg.d_model), 1.0 / math.sqrt(cfg.d_model)))
    return LayerInputs(cfg, x, wr, router_bias_values(cfg))
