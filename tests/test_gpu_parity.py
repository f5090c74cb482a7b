"""GPU parity at sizes the oracle finishes in seconds: every stage of the library against
the oracle on the same seeded inputs, over shapes that span several tiles and leave
ragged tails (rows per expert, output columns, K), plus the degenerate cases.

The structure of each reduced layer (gating, router skew recipe, capacity, shared
experts) is that of the named workload it shrinks.
"""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_29_amd import configs
from sparse_mixture_experts_29_amd.device import DeviceLayer
from sparse_mixture_experts_29_amd.inputs import make_inputs
import oracle
from tests import _parity as P

pytestmark = pytest.mark.gpu

R = configs.reduced
CASES = [
    configs.TINY_FP32,
    R(configs.TINY_FP32, T=333, d_model=192, d_ff=320),
    R(configs.MIXTRAL_PREFILL, T=1000, d_model=256, d_ff=384),
    R(configs.MIXTRAL_PREFILL, T=517, d_model=320, d_ff=576, n_experts=6, top_k=3),
    R(configs.QWEN3_FINE, T=777, d_model=256, d_ff=192, n_experts=32),
    R(configs.QWEN3_FINE_CF, T=777, d_model=256, d_ff=192, n_experts=32),
    R(configs.DEEPSEEK_V3, T=513, d_model=320, d_ff=128, n_experts=64, d_ff_shared=192),
    R(configs.DEEPSEEK_V3, T=200, d_model=256, d_ff=128, n_experts=300, top_k=8, n_shared=2,
      d_ff_shared=64),
    # decode batches: T = 1, 4, 16 on the weight-streaming kernels, T = 64 (16 rows per
    # expert) on the tiled GEMM
    *[R(configs.mixtral_decode(t), d_model=512, d_ff=1024) for t in (1, 4, 16, 64)],
    # small batches through the weight-streaming path, with a shared expert and a K tail
    R(configs.DEEPSEEK_V3, T=40, d_model=320, d_ff=192, n_experts=64, d_ff_shared=320),
    R(configs.QWEN3_FINE_CF, T=57, d_model=256, d_ff=128, n_experts=64, top_k=4),
    # the same with 16 experts: 14 rows per expert, so the tiled GEMM, capacity drops
    R(configs.QWEN3_FINE_CF, T=57, d_model=256, d_ff=128, n_experts=16, top_k=4),
    # tiled down launch with K split in two (d_ff >= 2 d_model), ragged tiles, with and
    # without a shared expert and capacity
    R(configs.MIXTRAL_PREFILL, T=600, d_model=256, d_ff=768),
    R(configs.DEEPSEEK_V3, T=300, d_model=128, d_ff=384, n_experts=16, top_k=4, d_ff_shared=256,
      capacity_factor=1.0),
    # decode-sized tiled batches (at most 16 rows per expert on average) on 64-row token tiles:
    # with a shared expert, with the split-K down launch, and ragged output widths
    R(configs.DEEPSEEK_V3, T=48, d_model=256, d_ff=192, n_experts=16, top_k=4, d_ff_shared=320),
    R(configs.DEEPSEEK_V3, T=60, d_model=128, d_ff=384, n_experts=16, top_k=4, d_ff_shared=256,
      capacity_factor=1.0),
    # small batches wide enough to split K in both launches (a 64-wide tail inside each split)
    R(configs.mixtral_decode(4), d_model=2176, d_ff=2176),
    R(configs.DEEPSEEK_V3, T=8, d_model=2048, d_ff=2048, n_experts=16, top_k=4, d_ff_shared=2048),
]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_stages_match_oracle(cfg):
    P.say(f"case {cfg}")
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    P.check_layer_full(li, dev)


EDGE = [
    # one expert: everything routes to it
    R(configs.MIXTRAL_PREFILL, T=130, d_model=128, d_ff=128, n_experts=1, top_k=1),
    # k = E: every token visits every expert (the dense mixture)
    R(configs.MIXTRAL_PREFILL, T=70, d_model=128, d_ff=256, n_experts=4, top_k=4),
    # tiny capacity: most pairs dropped, shared expert carries the dropped tokens
    R(configs.DEEPSEEK_V3, T=300, d_model=128, d_ff=128, n_experts=16, top_k=4, capacity_factor=0.1,
      d_ff_shared=128),
    # sigmoid with k = 1
    R(configs.DEEPSEEK_V3, T=129, d_model=128, d_ff=64, n_experts=8, top_k=1, n_shared=0),
    # a single token
    R(configs.QWEN3_FINE, T=1, d_model=128, d_ff=64, n_experts=128, top_k=8),
    # many experts with no tokens
    R(configs.QWEN3_FINE, T=3, d_model=128, d_ff=128, n_experts=1024, top_k=32),
    # route and permute in one launch: E <= 32 at T = 1 (sigmoid, shared expert; capacity 1)
    R(configs.DEEPSEEK_V3, T=1, d_model=256, d_ff=128, n_experts=32, top_k=4, d_ff_shared=128),
    R(configs.QWEN3_FINE_CF, T=1, d_model=128, d_ff=64, n_experts=16, top_k=2),
    # ... and E <= 8 with a partly filled 4-token block, bf16 and fp32
    R(configs.MIXTRAL_PREFILL, T=3, d_model=256, d_ff=128, n_experts=8, top_k=2),
    R(configs.TINY_FP32, T=2),
    # a single token with E <= 8, routed inside the gated launch, whose down launch combines:
    # sigmoid gates with a shared expert and capacity 1; k = E (every expert); one expert;
    # three shared experts (more waves per output chunk than the combined down launch takes)
    R(configs.DEEPSEEK_V3, T=1, d_model=256, d_ff=128, n_experts=8, top_k=3, d_ff_shared=128,
      capacity_factor=1.0),
    R(configs.MIXTRAL_PREFILL, T=1, d_model=192, d_ff=320, n_experts=4, top_k=4),
    R(configs.MIXTRAL_PREFILL, T=1, d_model=128, d_ff=192, n_experts=1, top_k=1),
    R(configs.DEEPSEEK_V3, T=1, d_model=128, d_ff=64, n_experts=6, top_k=6, n_shared=3, d_ff_shared=64),
]


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: c.name)
def test_edge_cases(cfg):
    P.say(f"case {cfg}")
    li = make_inputs(cfg)
    P.check_layer_full(li, DeviceLayer(li))


def test_collapsed_router_all_tokens_one_expert():
    """Zero router weights and a dominant bias: every token picks experts 3 then 0, 1, ..."""
    cfg = R(configs.MIXTRAL_PREFILL, T=300, d_model=128, d_ff=256, n_experts=8, top_k=2)
    li = make_inputs(cfg)
    li.w_router[:] = 0
    li.router_bias = np.zeros(8, np.float32)
    li.router_bias[3] = 5.0
    dev = DeviceLayer(li)
    b = dev.stage_buffers()
    dev.route(b)
    torch.cuda.synchronize()
    idx = P.host(b["idx"])
    assert (idx[:, 0] == 3).all() and (idx[:, 1] == 0).all()  # exact tie among the rest -> lowest
    P.check_layer_full(li, dev)


def test_capacity_with_collapsed_router_keeps_lowest_tokens():
    cfg = R(configs.QWEN3_FINE_CF, T=400, d_model=128, d_ff=128, n_experts=16, top_k=2)
    li = make_inputs(cfg)
    li.w_router[:] = 0
    li.router_bias = np.zeros(16, np.float32)
    li.router_bias[5] = 3.0
    dev = DeviceLayer(li)
    P.check_layer_full(li, dev)
    b = dev.stage_buffers()
    dev.route(b)
    dev.permute(b)
    torch.cuda.synchronize()
    C = int(np.ceil(1.25 * 400 * 2 / 16))
    keep = P.host(b["drop"]).reshape(400, 2)[:, 0] == 0  # slot 0 is expert 5 for every token
    assert keep[:C].all() and not keep[C:].any()


def test_layer_is_deterministic():
    cfg = R(configs.QWEN3_FINE, T=2000, d_model=256, d_ff=256, n_experts=64)
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    y1 = dev.forward().clone()
    ys = [dev.forward().clone() for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys:
        assert torch.equal(y, y1)


def test_stream_argument_is_honoured():
    cfg = R(configs.MIXTRAL_PREFILL, T=257, d_model=128, d_ff=128)
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    ref = dev.forward().clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    dev.y.zero_()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dev.forward(stream=s)
    s.synchronize()
    assert torch.equal(dev.y, ref)


def test_route_of_a_batch_large_enough_for_64_token_router_blocks():
    """T = 16384 with E = 256: the router takes 64-token blocks (T / 64 >= the CU count);
    expert sets, order, gates and logits against the oracle."""
    cfg = R(configs.DEEPSEEK_V3, T=16384, d_model=256, d_ff=64, n_experts=256, top_k=8, n_shared=0)
    P.say(f"case {cfg.name}")
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    b = dev.stage_buffers()
    dev.route(b)
    torch.cuda.synchronize()
    P.check_route(li, dev, b)


LDS_ROUTER = [
    # E not a multiple of 16 (part of the last 64-row block of W_r past E), one K block, ragged T
    R(configs.QWEN3_FINE, T=300, d_model=64, d_ff=64, n_experts=33, top_k=3),
    # sigmoid with a bias, E = 48, a two-block batch with a short last block
    R(configs.DEEPSEEK_V3, T=70, d_model=128, d_ff=64, n_experts=48, top_k=4, n_shared=0),
    # 128-row W_r blocks, three K blocks, 6 of 100
    R(configs.QWEN3_FINE, T=129, d_model=192, d_ff=64, n_experts=100, top_k=6),
    # 256-row W_r blocks (the three-stage ring), five K blocks
    R(configs.DEEPSEEK_V3, T=1000, d_model=320, d_ff=64, n_experts=200, top_k=8, n_shared=0),
    # 64-token blocks with a ragged last block of 5 tokens
    R(configs.DEEPSEEK_V3, T=16389, d_model=128, d_ff=64, n_experts=256, top_k=8, n_shared=0),
]


@pytest.mark.parametrize("cfg", LDS_ROUTER, ids=lambda c: c.name)
def test_router_with_operands_staged_through_lds(cfg):
    """The bf16 router for 32 < E <= 256 stages W_r and the token rows through LDS (E rounded
    up to a multiple of 64 rows, 64 k per stage, a ring of 3 to 8 stages): expert sets,
    order, gates and logits against the oracle across the shapes that change its layout."""
    P.say(f"case {cfg.name}")
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    b = dev.stage_buffers()
    dev.route(b)
    torch.cuda.synchronize()
    P.check_route(li, dev, b)


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (1024, 32)], ids=["small_e", "rows", "wave"])
def test_nan_logits_are_chosen_last_and_the_zeros_tie(E, k):
    """Each router path (E = 8: vector-ALU kernel; 128: MFMA logits, top-k on 16-lane rows;
    1024: top-k over whole waves) against the selection rule on non-finite and signed-zero
    logits, as the oracle's stable sort applies it (NaN sorts after every number). A token with
    a NaN activation has NaN logits everywhere: no larger logit decides, so it takes experts
    0..k-1 with NaN gates. A NaN bias makes that expert's logit NaN for every token: it is
    never chosen while k < E. On zero router weights the logits tie (zeros of either sign), so
    after the one expert with a positive bias the lower indices win. The other tokens route
    exactly as without the NaN."""
    P.say(f"case E={E} k={k}")
    cfg = R(configs.QWEN3_FINE, T=70, d_model=128, d_ff=64, n_experts=E, top_k=k, router_bias="none")
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    b = dev.stage_buffers()
    dev.route(b)
    torch.cuda.synchronize()
    idx0, gate0 = P.host(b["idx"]).copy(), P.host(b["gate"]).copy()

    nan_bf16 = torch.tensor([float("nan")], dtype=torch.bfloat16, device=dev.device)
    dev.x[5, 3] = nan_bf16[0]
    dev.route(b)
    torch.cuda.synchronize()
    idx, gate = P.host(b["idx"]), P.host(b["gate"])
    assert (idx[5] == np.arange(k)).all() and np.isnan(gate[5]).all()
    assert (oracle.select_topk(np.full((1, E), np.nan), k)[0] == np.arange(k)).all()
    rest = np.arange(cfg.T) != 5
    assert (idx[rest] == idx0[rest]).all() and np.array_equal(gate[rest], gate0[rest])

    bias = np.zeros(E, np.float32)
    bias[2] = np.nan
    dev.router_bias = torch.from_numpy(bias).to(dev.device)
    dev.route(b)
    torch.cuda.synchronize()
    assert not (P.host(b["idx"])[rest] == 2).any()
    one_nan = np.zeros((1, E))
    one_nan[0, 2] = np.nan
    assert 2 not in oracle.select_topk(one_nan, k)[0]

    dev.w_router.zero_()
    bias = np.zeros(E, np.float32)
    bias[1] = -0.0
    bias[4] = 1.0
    dev.router_bias = torch.from_numpy(bias).to(dev.device)
    dev.route(b)
    torch.cuda.synchronize()
    idx = P.host(b["idx"])
    want = np.array([4] + [e for e in range(E) if e != 4][: k - 1])
    assert (idx[rest] == want).all()
    assert (oracle.select_topk(bias[None, :].astype(np.float64), k)[0] == want).all()


def test_decode_tiles_collapsed_router_spans_several_tiles():
    """128 tokens, 16 experts, top-2 (8 rows per expert on average: 64-row token tiles), all
    routed to experts 9 then 0: two groups of 128 rows, two tiles each, the rest empty."""
    cfg = R(configs.MIXTRAL_PREFILL, T=128, d_model=256, d_ff=384, n_experts=16, top_k=2)
    li = make_inputs(cfg)
    li.w_router[:] = 0
    li.router_bias = np.zeros(16, np.float32)
    li.router_bias[9] = 4.0
    dev = DeviceLayer(li)
    P.check_layer_full(li, dev)


def test_small_batch_collapsed_router_fills_four_token_groups():
    """64 tokens all routed to expert 5 first: one group of 64 rows (4 groups of 16) on the
    weight-streaming kernels (32 experts: 4 rows per expert on average)."""
    cfg = R(configs.MIXTRAL_PREFILL, T=64, d_model=256, d_ff=512, n_experts=32, top_k=2)
    li = make_inputs(cfg)
    li.router_bias = np.zeros(32, np.float32)
    li.router_bias[5] = 4.0
    dev = DeviceLayer(li)
    P.check_layer_full(li, dev)
