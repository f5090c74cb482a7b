"""Problem statements of the MoE FFN layer forward and the named synthetic workloads.

A layer is described by the quantities the pages use for the problem: T tokens,
model width d, expert width f, E routed experts, top-k, the gating function
(softmax, or sigmoid renormalised over the chosen experts), a capacity factor
(<= 0 means dropless) and optional always-on shared experts ("Mixture of Experts",
shubhamtatvamasi.com, sections "The router" and "Load imbalance").

The named workloads are the five shapes this library is checked and measured on, plus
the decode shape with FP8 expert weights. They hold shapes and seeds only; the values
themselves come from ``inputs``.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

SOFTMAX = "softmax"
SIGMOID = "sigmoid"


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    gating: str = SOFTMAX
    capacity_factor: float = 0.0  # <= 0: dropless
    n_shared: int = 0
    d_ff_shared: int = 0
    dtype: str = "bf16"  # "f32" or "bf16": dtype of x, every weight, and y
    seed: int = 0
    router_bias: str = "none"  # "none" | "zipf" | "normal"
    bias_scale: float = 0.0  # zipf: exponent s; normal: std
    x_stream: int = 0  # index of x's random stream (decode sweeps use T)
    # expert weights: "dtype" (stored in `dtype`) or "fp8_e4m3" (one-byte E4M3 codes and one
    # float32 scale per output row; activations and the router stay in `dtype`)
    weights: str = "dtype"

    @property
    def dropless(self) -> bool:
        return not (self.capacity_factor > 0)

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    # --- algorithmic accounting (two FLOPs per multiply-add) -------------
    def expert_flops_per_pair(self) -> int:
        """gate, up and down projections of one routed (token, expert) pair."""
        return 6 * self.d_model * self.d_ff

    def shared_flops(self) -> int:
        return 6 * self.d_model * self.d_ff_shared * self.T * self.n_shared

    def router_flops(self) -> int:
        return 2 * self.T * self.d_model * self.n_experts

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def fp8(self) -> bool:
        return self.weights == "fp8_e4m3"

    def matrix_bytes(self, rows: int, cols: int) -> int:
        """Stored bytes of one expert matrix with `rows` output rows (codes + row scales for
        FP8 weights)."""
        if self.fp8:
            return rows * cols + 4 * rows
        return rows * cols * self.elem_bytes

    def gate_up_bytes(self, f: int) -> int:
        """gate and up matrices of one expert of width f."""
        return 2 * self.matrix_bytes(f, self.d_model)

    def down_bytes(self, f: int) -> int:
        return self.matrix_bytes(self.d_model, f)

    def expert_weight_bytes(self) -> int:
        return self.gate_up_bytes(self.d_ff) + self.down_bytes(self.d_ff)

    def total_weight_bytes(self) -> int:
        b = self.n_experts * self.expert_weight_bytes()
        b += self.n_shared * (self.gate_up_bytes(self.d_ff_shared) + self.down_bytes(self.d_ff_shared))
        b += self.n_experts * self.d_model * self.elem_bytes
        return b


# Tiny fp32 layer: T=64, d=128, f=256, E=8, top-2, softmax, dropless.
TINY_FP32 = LayerConfig("tiny_fp32_T64_d128_f256_E8_k2", T=64, d_model=128, d_ff=256,
                        n_experts=8, top_k=2, dtype="f32", seed=0)
# Mixtral-shaped prefill: T=4096, d=4096, f=14336, E=8, top-2, softmax, bf16.
MIXTRAL_PREFILL = LayerConfig("mixtral_prefill_T4096_d4096_f14336_E8_k2", T=4096, d_model=4096,
                              d_ff=14336, n_experts=8, top_k=2, seed=1)


def mixtral_decode(T: int) -> LayerConfig:
    """Mixtral-shaped low-batch decode layer; T in {1, 4, 16, 64} tokens per step."""
    return LayerConfig(f"mixtral_decode_T{T}_d4096_f14336_E8_k2", T=T, d_model=4096,
                       d_ff=14336, n_experts=8, top_k=2, seed=2, x_stream=T)


DECODE_TS = (1, 4, 16, 64)


def mixtral_decode_fp8(T: int) -> LayerConfig:
    """The Mixtral-shaped decode layer with FP8 E4M3 expert weights (per-row scales); the
    codes quantise the same draws as mixtral_decode(T)'s weights."""
    return mixtral_decode(T).replace(name=f"mixtral_decode_fp8_T{T}_d4096_f14336_E8_k2", weights="fp8_e4m3")


# Fine-grained Qwen3-30B-A3B-style layer: T=8192, d=2048, f=768, E=128, top-8, Zipf-skewed
# router bias; run dropless and with capacity factor 1.25.
QWEN3_FINE = LayerConfig("qwen3_fine_T8192_d2048_f768_E128_k8", T=8192, d_model=2048, d_ff=768,
                         n_experts=128, top_k=8, seed=3, router_bias="zipf", bias_scale=1.1)
QWEN3_FINE_CF = QWEN3_FINE.replace(name="qwen3_fine_cf1.25_T8192_d2048_f768_E128_k8",
                                   capacity_factor=1.25)
# DeepSeek-V3-style layer: T=16384, d=7168, f=2048, E=256, top-8, sigmoid, 1 shared expert.
DEEPSEEK_V3 = LayerConfig("deepseek_v3_T16384_d7168_f2048_E256_k8_s1", T=16384, d_model=7168,
                          d_ff=2048, n_experts=256, top_k=8, gating=SIGMOID, n_shared=1,
                          d_ff_shared=2048, seed=4, router_bias="normal", bias_scale=0.5)

ALL = {c.name: c for c in [TINY_FP32, MIXTRAL_PREFILL, *[mixtral_decode(t) for t in DECODE_TS],
                           QWEN3_FINE, QWEN3_FINE_CF, DEEPSEEK_V3,
                           *[mixtral_decode_fp8(t) for t in DECODE_TS]]}


@dataclasses.dataclass(frozen=True)
class ShardWorkload:
    """One GPU's share of an expert-parallel layer: `layer` routed over all its experts
    (global T tokens), the GPU owning experts [shard*E/n, (shard+1)*E/n) runs the rows routed
    there (moe_expert_shard_forward)."""
    name: str
    layer: LayerConfig
    n_shards: int
    shard: int


SHARDS = {w.name: w for w in [
    ShardWorkload("deepseek_v3_ep8_shard0_T16384_d7168_f2048_E256_k8", DEEPSEEK_V3, 8, 0),
    ShardWorkload("qwen3_fine_ep8_shard0_T8192_d2048_f768_E128_k8", QWEN3_FINE, 8, 0),
    ShardWorkload("mixtral_prefill_ep8_shard0_T4096_d4096_f14336_E8_k2", MIXTRAL_PREFILL, 8, 0),
]}


def reduced(cfg: LayerConfig, **kw) -> LayerConfig:
    """Same structure (gating, skew recipe, shared experts, capacity) at a smaller size."""
    name = cfg.name.split("_T")[0] + "_reduced_" + "_".join(f"{k}{v}" for k, v in sorted(kw.items()))
    return cfg.replace(name=name, **kw)
