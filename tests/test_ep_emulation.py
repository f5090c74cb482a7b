"""Expert parallelism emulated on the CPU: P processes (gloo, 127.0.0.1) each own T/P tokens
and E/P experts, and one layer step runs as the sharding design lays it out -- local route,
an all-to-all of per-destination row counts, a dispatch all-to-allv of the token rows, each
rank's experts on the rows it received (capacity applied in receive order), a combine
all-to-allv back, and the gate-weighted sum (plus the shared experts) at home. The result must
equal the one-process oracle layer on every token.

Pages: shubhamtatvamasi.com/llm-inference/moe, section on expert parallelism (whole experts
live on different GPUs; each token's rows are sent to the GPUs owning its experts, and the
results come back to the token's home GPU to be weighted by the gate); klaylearn.com/glossary/
mixture-of-experts, definition (permute by destination, grouped GEMM, undo the permutation).

All arithmetic is the oracle's (float64); the bookkeeping under test is the row order of
device.shard_rows (ascending token, then slot, sources in rank order), which is the order the
expert-parallel shard entry point expects, and the capacity rule it implies: with sources
holding contiguous token ranges in rank order, the receive order of an expert's rows is
ascending global token, so keeping the first C received rows keeps the same pairs as the
one-GPU layer.
"""
import os
import socket

import numpy as np
import pytest
import torch
import torch.distributed as dist
import torch.multiprocessing as mp

import oracle
from sparse_mixture_experts_29_amd import configs
from sparse_mixture_experts_29_amd.device import shard_rows
from sparse_mixture_experts_29_amd.inputs import make_inputs

R = configs.reduced


def _a2a(send: torch.Tensor, send_counts, recv_counts) -> torch.Tensor:
    out = torch.empty((int(sum(recv_counts)),) + tuple(send.shape[1:]), dtype=send.dtype)
    dist.all_to_all_single(out, send.contiguous(), [int(v) for v in recv_counts], [int(v) for v in send_counts])
    return out


def _rank_main(rank: int, P: int, port: int, cfg, out_dir: str):
    dist.init_process_group("gloo", init_method=f"tcp://127.0.0.1:{port}", rank=rank, world_size=P)
    try:
        c = cfg
        li = make_inputs(c)
        E, per, Tl, d = c.n_experts, c.n_experts // P, c.T // P, c.d_model
        x_all = li.values(li.x).astype(np.float64)
        t0 = rank * Tl
        x = x_all[t0:t0 + Tl]
        # 1. local route
        idx, gate, _ = oracle.route(x, li.values(li.w_router), li.router_bias, c.top_k, c.gating)
        # 2. per-destination rows (ascending token, then slot) and the count exchange
        rows = [shard_rows(idx, P, p, E) for p in range(P)]
        send_counts = torch.tensor([len(r[0]) for r in rows], dtype=torch.int64)
        recv_counts = torch.empty(P, dtype=torch.int64)
        dist.all_to_all_single(recv_counts, send_counts)
        # 3. dispatch all-to-allv: the token rows and their local expert ids
        send_x = torch.from_numpy(np.concatenate([x[r[0]] for r in rows]))
        send_e = torch.from_numpy(np.concatenate([r[2] for r in rows]).astype(np.int64))
        recv_x = _a2a(send_x, send_counts, recv_counts).numpy()
        recv_e = _a2a(send_e, send_counts, recv_counts).numpy()
        # 4. this rank's experts on the received rows; capacity C (of the whole layer) keeps each
        # expert's first C rows in receive order = ascending global token
        cap = oracle.expert_capacity(c.capacity_factor, c.T, c.top_k, E)
        y_recv = np.zeros_like(recv_x)
        keep = np.ones(len(recv_e), bool)
        for el in range(per):
            m = np.flatnonzero(recv_e == el)
            if cap is not None:
                keep[m[cap:]] = False
                m = m[:cap]
            if m.size:
                y_recv[m] = oracle.swiglu_ffn(recv_x[m], *li.expert_values(rank * per + el))
        # 5. combine all-to-allv back to the home ranks (rows return in the order they were sent)
        back = _a2a(torch.from_numpy(y_recv), recv_counts, send_counts).numpy()
        back_keep = _a2a(torch.from_numpy(keep.astype(np.int64)), recv_counts, send_counts).numpy()
        # 6. gate-weighted sum at home, plus the shared experts on the home tokens
        y = np.zeros((Tl, d))
        tok = np.concatenate([r[0] for r in rows])
        slot = np.concatenate([r[1] for r in rows])
        for j in range(c.top_k):  # slot order, as the one-GPU combine sums
            m = (slot == j) & (back_keep == 1)
            y[tok[m]] += gate[tok[m], j, None] * back[m]
        if c.n_shared:
            y += oracle.shared_mlp(x, lambda s: li.shared_values(s), c.n_shared).sum(axis=0)
        np.save(os.path.join(out_dir, f"y{rank}.npy"), y)
        np.save(os.path.join(out_dir, f"drop{rank}.npy"), 1 - back_keep)
    finally:
        dist.destroy_process_group()


def _free_port() -> int:
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


@pytest.mark.parametrize("cfg,P", [
    (R(configs.DEEPSEEK_V3, T=96, d_model=64, d_ff=64, n_experts=16, d_ff_shared=64), 2),
    (R(configs.DEEPSEEK_V3, T=96, d_model=64, d_ff=64, n_experts=16, d_ff_shared=64), 4),
    (R(configs.QWEN3_FINE_CF, T=128, d_model=64, d_ff=64, n_experts=32), 4),
    (R(configs.MIXTRAL_PREFILL, T=64, d_model=64, d_ff=128), 2),
], ids=lambda v: getattr(v, "name", str(v)))
def test_expert_parallel_round_trip_equals_one_process_layer(tmp_path, cfg, P):
    assert cfg.T % P == 0 and cfg.n_experts % P == 0
    mp.spawn(_rank_main, args=(P, _free_port(), cfg, str(tmp_path)), nprocs=P, join=True)
    li = make_inputs(cfg)
    ref = oracle.forward(li.values(li.x), li.values(li.w_router), li.router_bias, top_k=cfg.top_k, gating=cfg.gating,
                         capacity_factor=cfg.capacity_factor, experts=lambda e: li.expert_values(e),
                         shared=lambda s: li.shared_values(s), n_shared=cfg.n_shared)
    y = np.concatenate([np.load(tmp_path / f"y{r}.npy") for r in range(P)])
    np.testing.assert_allclose(y, ref["y"], rtol=1e-12, atol=1e-12)
    # the drops at the owners are exactly the one-GPU layer's drops
    Tl = cfg.T // P
    n_drop = sum(int(np.load(tmp_path / f"drop{r}.npy").sum()) for r in range(P))
    assert n_drop == int(ref["drop"].sum())
    if cfg.capacity_factor > 0:
        assert n_drop > 0, "the capacity case should drop pairs"
    assert Tl * P == cfg.T
