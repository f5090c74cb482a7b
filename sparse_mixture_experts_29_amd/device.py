"""Device-resident layer: uploads a layer's inputs once and owns its outputs and workspace.

Plumbing for callers of the binding (tests, benchmark, smoke run): torch allocates the
device memory, the library computes. Weights are uploaded expert by expert while other
threads draw the next experts, so a 22.6 GB layer never sits whole in host memory.
"""
from __future__ import annotations

import threading
from typing import Optional

import numpy as np
import torch

from . import binding
from .configs import LayerConfig
from .inputs import LayerInputs


def torch_dtype(cfg: LayerConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def host_to_device(a: np.ndarray, cfg: LayerConfig, device) -> torch.Tensor:
    """Upload a storage array (uint16 bf16 bits or float32) as a bf16/fp32 device tensor."""
    if cfg.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def device_to_host_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


class DeviceLayer:
    def __init__(self, li: LayerInputs, device: str = "cuda:0", threads: int = 8,
                 weights_from: Optional["DeviceLayer"] = None):
        """weights_from: reuse the expert weights already uploaded for another layer of the
        same shape and seed (e.g. the same layer at another token count)."""
        cfg = li.cfg
        self.cfg, self.inputs, self.device = cfg, li, torch.device(device)
        dt = torch_dtype(cfg)
        E, d, f = cfg.n_experts, cfg.d_model, cfg.d_ff
        self.x = host_to_device(li.x, cfg, device)
        self.w_router = host_to_device(li.w_router, cfg, device)
        self.router_bias = None if li.router_bias is None else torch.from_numpy(li.router_bias).to(device)
        self.s_gate = self.s_up = self.s_down = None  # FP8 row scales
        self.ss_gate = self.ss_up = self.ss_down = None
        if weights_from is not None:
            o = weights_from.cfg
            assert (o.seed, o.n_experts, o.d_model, o.d_ff, o.dtype, o.weights) == \
                (cfg.seed, E, d, f, cfg.dtype, cfg.weights)
            self.w_gate, self.w_up, self.w_down = weights_from.w_gate, weights_from.w_up, weights_from.w_down
            self.s_gate, self.s_up, self.s_down = weights_from.s_gate, weights_from.s_up, weights_from.s_down
        elif cfg.fp8:
            self.w_gate, self.w_up, self.w_down, self.s_gate, self.s_up, self.s_down = \
                _upload_fp8(li, E, f, d, device, threads, shared=False)
        else:
            self.w_gate = torch.empty((E, f, d), dtype=dt, device=device)
            self.w_up = torch.empty((E, f, d), dtype=dt, device=device)
            self.w_down = torch.empty((E, d, f), dtype=dt, device=device)
            lock = threading.Lock()

            def put(e, w):
                with lock:
                    self.w_gate[e].copy_(host_to_device(w[0], cfg, device))
                    self.w_up[e].copy_(host_to_device(w[1], cfg, device))
                    self.w_down[e].copy_(host_to_device(w[2], cfg, device))

            li.for_each_expert(put, threads)
        self.ws_gate = self.ws_up = self.ws_down = None
        if cfg.n_shared and cfg.fp8:
            self.ws_gate, self.ws_up, self.ws_down, self.ss_gate, self.ss_up, self.ss_down = \
                _upload_fp8(li, cfg.n_shared, cfg.d_ff_shared, d, device, 1, shared=True)
        elif cfg.n_shared:
            fs = cfg.d_ff_shared
            self.ws_gate = torch.empty((cfg.n_shared, fs, d), dtype=dt, device=device)
            self.ws_up = torch.empty((cfg.n_shared, fs, d), dtype=dt, device=device)
            self.ws_down = torch.empty((cfg.n_shared, d, fs), dtype=dt, device=device)
            for s in range(cfg.n_shared):
                w = li.shared(s)
                self.ws_gate[s].copy_(host_to_device(w[0], cfg, device))
                self.ws_up[s].copy_(host_to_device(w[1], cfg, device))
                self.ws_down[s].copy_(host_to_device(w[2], cfg, device))
        self.y = torch.empty((cfg.T, d), dtype=dt, device=device)
        self.ws = torch.empty(binding.moe_workspace_size(cfg, binding.MOE_OP_LAYER), dtype=torch.uint8,
                              device=device)
        torch.cuda.synchronize(self.device)

    def fp8_experts(self):
        """The routed and shared moe_fp8_weights of an FP8 layer (shared None without)."""
        ex = binding.fp8_weights((self.w_gate, self.w_up, self.w_down, self.s_gate, self.s_up, self.s_down))
        sh = None
        if self.cfg.n_shared:
            sh = binding.fp8_weights((self.ws_gate, self.ws_up, self.ws_down, self.ss_gate, self.ss_up,
                                      self.ss_down))
        return ex, sh

    # ---------------------------------------------------------------- whole layer
    def forward(self, stream=None) -> torch.Tensor:
        if self.cfg.fp8:
            ex, sh = self.fp8_experts()
            binding.moe_layer_forward_fp8(self.cfg, self.x, self.w_router, self.router_bias, ex, sh, self.y,
                                          self.ws, stream)
            return self.y
        binding.moe_layer_forward(self.cfg, self.x, self.w_router, self.router_bias, self.w_gate,
                                  self.w_up, self.w_down, self.ws_gate, self.ws_up, self.ws_down,
                                  self.y, self.ws, stream)
        return self.y

    def backward(self, dy: torch.Tensor, aux_coef: float = 0.0, grads: Optional["LayerGrads"] = None,
                 stream=None) -> "LayerGrads":
        """moe_layer_backward for the output gradient dy [T][d]; returns the gradient buffers."""
        g = grads if grads is not None else LayerGrads(self)
        binding.moe_layer_backward(self.cfg, self.x, self.w_router, self.router_bias, self.w_gate, self.w_up,
                                   self.w_down, self.ws_gate, self.ws_up, self.ws_down, dy, aux_coef, g.struct, g.ws,
                                   stream)
        return g

    # ---------------------------------------------------------------- step by step
    def stage_buffers(self) -> dict:
        cfg, dev = self.cfg, self.device
        pairs = cfg.T * cfg.top_k
        mk = binding.moe_max_kept(cfg)
        dt = torch_dtype(cfg)
        b = dict(
            idx=torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device=dev),
            gate=torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device=dev),
            logits=torch.empty((cfg.T, cfg.n_experts), dtype=torch.float32, device=dev),
            counts=torch.empty(cfg.n_experts, dtype=torch.int32, device=dev),
            offsets=torch.empty(cfg.n_experts + 1, dtype=torch.int32, device=dev),
            sorted_slot=torch.empty(mk, dtype=torch.int32, device=dev),
            pos=torch.empty(pairs, dtype=torch.int32, device=dev),
            drop=torch.empty(pairs, dtype=torch.uint8, device=dev),
            permute_ws=torch.empty(max(1, binding.moe_workspace_size(cfg, binding.MOE_OP_PERMUTE)),
                                   dtype=torch.uint8, device=dev),
            grouped_ws=torch.empty(max(1, binding.moe_workspace_size(cfg, binding.MOE_OP_GROUPED_MLP)),
                                   dtype=torch.uint8, device=dev),
            # rows past N_kept (capacity mode) are never written: zeros, not leftovers
            y_perm=torch.zeros((mk, cfg.d_model), dtype=dt, device=dev),
            y_shared=(torch.empty((cfg.n_shared, cfg.T, cfg.d_model), dtype=dt, device=dev)
                      if cfg.n_shared else None),
            y=torch.empty((cfg.T, cfg.d_model), dtype=dt, device=dev),
        )
        return b

    def route(self, b: dict, logits: bool = True, stream=None):
        binding.moe_route(self.cfg, self.x, self.w_router, self.router_bias, b["idx"], b["gate"],
                          b["logits"] if logits else None, stream)

    def permute(self, b: dict, idx: Optional[torch.Tensor] = None, stream=None):
        binding.moe_permute(self.cfg, b["idx"] if idx is None else idx, b["counts"], b["offsets"],
                            b["sorted_slot"], b["pos"], b["drop"], b["permute_ws"], stream)

    def grouped_mlp(self, b: dict, stream=None):
        if self.cfg.fp8:
            ex, sh = self.fp8_experts()
            binding.moe_grouped_mlp_fp8(self.cfg, self.x, b["sorted_slot"], b["offsets"], ex, sh, b["y_perm"],
                                        b["y_shared"], b["grouped_ws"], stream)
            return
        binding.moe_grouped_mlp(self.cfg, self.x, b["sorted_slot"], b["offsets"], self.w_gate, self.w_up,
                                self.w_down, self.ws_gate, self.ws_up, self.ws_down, b["y_perm"],
                                b["y_shared"], b["grouped_ws"], stream)

    def combine(self, b: dict, stream=None):
        binding.moe_combine(self.cfg, b["y_perm"], b["pos"], b["gate"], b["y_shared"], b["y"], stream)


class LayerGrads:
    """Device buffers for the gradients of a DeviceLayer (moe_layer_backward) and the
    backward workspace."""

    def __init__(self, layer: "DeviceLayer"):
        cfg, dev = layer.cfg, layer.device
        dt = torch_dtype(cfg)
        E, d, f = cfg.n_experts, cfg.d_model, cfg.d_ff
        self.dx = torch.empty((cfg.T, d), dtype=dt, device=dev)
        self.dw_router = torch.empty((E, d), dtype=dt, device=dev)
        self.d_router_bias = torch.empty(E, dtype=torch.float32, device=dev)
        self.dw_gate = torch.empty((E, f, d), dtype=dt, device=dev)
        self.dw_up = torch.empty((E, f, d), dtype=dt, device=dev)
        self.dw_down = torch.empty((E, d, f), dtype=dt, device=dev)
        self.dws_gate = self.dws_up = self.dws_down = None
        if cfg.n_shared:
            fs = cfg.d_ff_shared
            self.dws_gate = torch.empty((cfg.n_shared, fs, d), dtype=dt, device=dev)
            self.dws_up = torch.empty((cfg.n_shared, fs, d), dtype=dt, device=dev)
            self.dws_down = torch.empty((cfg.n_shared, d, fs), dtype=dt, device=dev)
        self.aux_loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.ws = torch.empty(binding.moe_workspace_size(cfg, binding.MOE_OP_LAYER_BACKWARD), dtype=torch.uint8,
                              device=dev)
        self.struct = binding.layer_grads(self.dx, self.dw_router, self.d_router_bias, self.dw_gate, self.dw_up,
                                          self.dw_down, self.dws_gate, self.dws_up, self.dws_down, self.aux_loss)


def _upload_fp8(li: LayerInputs, n: int, f: int, d: int, device, threads: int, shared: bool):
    """Codes (uint8) and row scales (float32) of n FP8 experts of width f, uploaded one expert
    at a time: gate, up [n][f][d], down [n][d][f], scales [n][f], [n][f], [n][d]."""
    u8 = dict(dtype=torch.uint8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    t = [torch.empty((n, f, d), **u8), torch.empty((n, f, d), **u8), torch.empty((n, d, f), **u8),
         torch.empty((n, f), **f32), torch.empty((n, f), **f32), torch.empty((n, d), **f32)]
    lock = threading.Lock()

    def put(e, w):
        with lock:
            for dst, src in zip(t, w):
                dst[e].copy_(torch.from_numpy(np.ascontiguousarray(src)))

    li.for_each_expert(put, threads, shared=shared)
    return tuple(t)


def shard_rows(idx, n_shards: int, shard: int, n_experts: int):
    """The rows the GPU owning shard `shard` of an expert-parallel layer receives: every
    (token, slot) pair whose expert lies in that shard's contiguous range of E / n_shards
    experts, in source order (home GPUs own contiguous token ranges), then token, then slot.
    Returns (token, slot, local expert id) arrays."""
    per = n_experts // n_shards
    idx = np.asarray(idx)
    tok, slot = np.nonzero(idx // per == shard)  # row-major: ascending token, then slot
    return tok, slot, (idx[tok, slot] - shard * per).astype(np.int32)


class ExpertShard:
    """One shard of an expert-parallel layer on this GPU: the received rows, their local
    expert ids and the shard's expert weights; forward() runs moe_expert_shard_forward.
    Build it from a DeviceLayer (views of its weights) or from seeded inputs (only the
    shard's experts are generated and uploaded)."""

    def __init__(self, cfg: LayerConfig, n_shards: int, shard: int, x, w_gate, w_up, w_down, tok, local_expert):
        per = cfg.n_experts // n_shards
        dev = x.device
        self.tok = torch.as_tensor(tok, dtype=torch.int64, device=dev)
        self.local_expert = torch.as_tensor(local_expert, dtype=torch.int32, device=dev)
        R = int(self.tok.numel())
        self.cfg = cfg.replace(name=f"{cfg.name}_shard{shard}of{n_shards}", T=R, n_experts=per, top_k=1,
                               capacity_factor=0.0, n_shared=0, d_ff_shared=0)
        self.x_recv = x.index_select(0, self.tok).contiguous()
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        self.y_send = torch.empty_like(self.x_recv)
        self.ws = torch.empty(max(binding.moe_workspace_size(self.cfg, binding.MOE_OP_LAYER), 1), dtype=torch.uint8,
                              device=dev)

    @classmethod
    def from_layer(cls, layer: DeviceLayer, n_shards: int, shard: int, tok, local_expert) -> "ExpertShard":
        per = layer.cfg.n_experts // n_shards
        e0 = shard * per
        return cls(layer.cfg, n_shards, shard, layer.x, layer.w_gate[e0:e0 + per], layer.w_up[e0:e0 + per],
                   layer.w_down[e0:e0 + per], tok, local_expert)

    @classmethod
    def from_inputs(cls, li: LayerInputs, n_shards: int, shard: int, x, tok, local_expert, threads: int = 8):
        cfg = li.cfg
        per = cfg.n_experts // n_shards
        dt = torch_dtype(cfg)
        d, f = cfg.d_model, cfg.d_ff
        wg = torch.empty((per, f, d), dtype=dt, device=x.device)
        wu = torch.empty((per, f, d), dtype=dt, device=x.device)
        wd = torch.empty((per, d, f), dtype=dt, device=x.device)

        def put(i):
            w = li.expert(shard * per + i)
            wg[i].copy_(host_to_device(w[0], cfg, x.device))
            wu[i].copy_(host_to_device(w[1], cfg, x.device))
            wd[i].copy_(host_to_device(w[2], cfg, x.device))

        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max(1, threads)) as ex:
            list(ex.map(put, range(per)))
        return cls(cfg, n_shards, shard, x, wg, wu, wd, tok, local_expert)

    def forward(self, stream=None):
        binding.moe_expert_shard_forward(self.cfg, self.x_recv, self.local_expert, self.w_gate, self.w_up,
                                         self.w_down, self.y_send, self.ws, stream)
        return self.y_send
