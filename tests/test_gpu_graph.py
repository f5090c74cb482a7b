"""HIP graph capture of the layer entry points.

moe_layer_forward (weight-streaming and tiled paths, shared experts, capacity),
moe_layer_forward_fp8 and moe_layer_backward enqueue nothing but kernel launches on the
caller's stream: no memset, no copy, no synchronisation, no allocation. So a call captured
with torch.cuda.CUDAGraph (a HIP graph on ROCm) replays as a unit. Every replay, each after
eager work of the program's own and a synchronisation, with the outputs poisoned before it,
must reproduce the eager result bit for bit: the kernels are deterministic.

Pages: shubhamtatvamasi.com/llm-inference/moe, "Memory vs compute, quantified" (decode steps
are short and repeated; launch overhead counts there).
"""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_29_amd import configs
from sparse_mixture_experts_29_amd.device import DeviceLayer, LayerGrads
from sparse_mixture_experts_29_amd.inputs import make_inputs, output_grad
from tests import _parity as P

pytestmark = pytest.mark.gpu

R = configs.reduced

FORWARD_CASES = [
    # weight-streaming kernels, combine from their split-K partials
    R(configs.mixtral_decode(1), d_model=512, d_ff=1024),
    # tiled GEMM with the down launch's K split in two, combine from the partials
    R(configs.MIXTRAL_PREFILL, T=600, d_model=256, d_ff=768),
    # tiled GEMM, unsplit down launch, shared expert, capacity drops
    R(configs.DEEPSEEK_V3, T=300, d_model=128, d_ff=192, n_experts=16, top_k=4, d_ff_shared=256,
      capacity_factor=1.0),
    # FP8 expert weights
    R(configs.mixtral_decode_fp8(4), d_model=512, d_ff=1024),
]

REPLAYS = 4


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _eager_work(n: int):
    """Unrelated work of the program between replays (fp32, so no batched bf16 products)."""
    a = torch.randn((256, 256), device="cuda:0", generator=torch.Generator("cuda:0").manual_seed(n))
    return float((a @ a).sum().item())


def _capture(fn):
    """Warm up on a side stream, then capture one call of fn into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("cfg", FORWARD_CASES, ids=lambda c: c.name)
def test_forward_graph_replays_equal_the_eager_call(cfg):
    P.say(f"case {cfg.name}")
    dev = DeviceLayer(make_inputs(cfg))
    ref = dev.forward().clone()
    torch.cuda.synchronize()
    g = _capture(dev.forward)
    for rep in range(REPLAYS):
        dev.y.fill_(float("nan"))
        _eager_work(rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dev.y, ref), f"replay {rep}: max diff {(dev.y.float() - ref.float()).abs().max().item()}"
    # the captured call reads x when replayed, not when captured (negated x: other routing)
    dev.x.neg_()
    torch.cuda.synchronize()
    eager_neg = dev.forward().clone()
    dev.y.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(dev.y, eager_neg)
    assert not torch.equal(eager_neg, ref)


def test_backward_graph_replays_equal_the_eager_call():
    cfg = R(configs.MIXTRAL_PREFILL, T=300, d_model=256, d_ff=384)
    P.say(f"case {cfg.name}")
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    dy = torch.from_numpy(output_grad(cfg).view(np.int16)).view(torch.bfloat16).to(dev.device)
    grads = LayerGrads(dev)
    names = ["dx", "dw_router", "d_router_bias", "dw_gate", "dw_up", "dw_down", "aux_loss"]
    dev.backward(dy, aux_coef=0.01, grads=grads)
    torch.cuda.synchronize()
    ref = {n: getattr(grads, n).clone() for n in names}
    g = _capture(lambda: dev.backward(dy, aux_coef=0.01, grads=grads))
    for rep in range(REPLAYS):
        for n in names:
            getattr(grads, n).fill_(float("nan"))
        _eager_work(100 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(grads, n), ref[n]), f"replay {rep}: {n}"
