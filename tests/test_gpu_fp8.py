"""GPU parity of the FP8 expert weights path (moe_grouped_mlp_fp8, moe_layer_forward_fp8):
every stage against the oracle, whose weights are the codes decoded from the E4M3 definition
times the row scales, on decode-sized batches with several K blocks, split K with a 64-wide
tail, shared experts and capacity; and, with power-of-two scales, bit-identical results to
the bf16 path run on the same weight values (an E4M3 value times a power of two is a bf16
value, and the FP8 kernels multiply in the same order).

Pages: shubhamtatvamasi.com/llm-inference/moe, "Memory vs compute, quantified" (FP8 weights
at half the bytes; decode reads the touched experts' weights).
"""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_29_amd import configs
from sparse_mixture_experts_29_amd.device import DeviceLayer
from sparse_mixture_experts_29_amd.inputs import make_inputs
from tests import _parity as P

pytestmark = pytest.mark.gpu

R = configs.reduced


def fp8(cfg):
    return cfg.replace(name=cfg.name.replace("_T", "_fp8_T", 1), weights="fp8_e4m3")


CASES = [
    *[R(configs.mixtral_decode_fp8(t), d_model=512, d_ff=1024) for t in configs.DECODE_TS],
    # K split in both launches, a 64-wide tail inside each split
    R(configs.mixtral_decode_fp8(4), d_model=2176, d_ff=2176),
    # a shared FP8 expert beside the routed ones, K split
    R(fp8(configs.DEEPSEEK_V3), T=8, d_model=2048, d_ff=2048, n_experts=16, top_k=4, d_ff_shared=2048),
    # a shared expert wider than the routed ones, two token groups per wave
    R(fp8(configs.DEEPSEEK_V3), T=40, d_model=320, d_ff=192, n_experts=64, d_ff_shared=320),
    # capacity with drops (14 rows per expert: the bf16 layer would take the tiled GEMM)
    R(fp8(configs.QWEN3_FINE_CF), T=57, d_model=256, d_ff=128, n_experts=16, top_k=4),
    # one token, many experts
    R(fp8(configs.QWEN3_FINE), T=1, d_model=128, d_ff=64, n_experts=128, top_k=8),
    # capacity with drops, 4 rows per expert (the bf16 layer runs the same kernels)
    R(fp8(configs.QWEN3_FINE_CF), T=57, d_model=256, d_ff=128, n_experts=64, top_k=4),
    # a single token with E <= 8, routed inside the gated launch: sigmoid gates with a shared
    # expert and capacity 1; k = E
    R(fp8(configs.DEEPSEEK_V3), T=1, d_model=256, d_ff=128, n_experts=8, top_k=3, d_ff_shared=128,
      capacity_factor=1.0),
    R(configs.mixtral_decode_fp8(1), d_model=192, d_ff=320, n_experts=4, top_k=4),
    # a single token whose down units do not fit one block (8 experts and a shared one): two
    # chunks a wave and the combine as a launch of its own
    R(fp8(configs.DEEPSEEK_V3), T=1, d_model=2304, d_ff=256, n_experts=64, top_k=8, d_ff_shared=256),
]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_fp8_stages_match_oracle(cfg):
    P.say(f"case {cfg}")
    li = make_inputs(cfg)
    P.check_layer_full(li, DeviceLayer(li))


def _pow2(s: torch.Tensor) -> torch.Tensor:
    return torch.exp2(torch.round(torch.log2(s)))


# cases whose bf16 layer also runs on the weight-streaming kernels (fewer than 8 rows per expert)
@pytest.mark.parametrize("cfg", [CASES[1], CASES[4], CASES[5], CASES[9]], ids=lambda c: c.name)
def test_fp8_with_power_of_two_scales_equals_the_bf16_path_bitwise(cfg):
    P.say(f"case {cfg.name}")
    li8 = make_inputs(cfg)
    d8 = DeviceLayer(li8)
    # scales rounded to powers of two: every dequantised weight is exactly a bf16 value
    for name in ("s_gate", "s_up", "s_down", "ss_gate", "ss_up", "ss_down"):
        t = getattr(d8, name)
        if t is not None:
            t.copy_(_pow2(t))
    li16 = make_inputs(cfg.replace(weights="dtype"))
    d16 = DeviceLayer(li16)
    pairs = [("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down")]
    if cfg.n_shared:
        pairs += [("ws_gate", "ss_gate"), ("ws_up", "ss_up"), ("ws_down", "ss_down")]
    for w, s in pairs:
        codes = getattr(d8, w).cpu()
        scale = getattr(d8, s).cpu()
        vals = codes.view(torch.float8_e4m3fn).to(torch.float32) * scale[:, :, None]
        exact = vals.to(torch.bfloat16)
        assert torch.equal(exact.to(torch.float32), vals)
        getattr(d16, w).copy_(exact.to(d16.device))
    torch.cuda.synchronize()
    y8 = d8.forward().clone()
    y16 = d16.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(y8, y16), f"max diff {(y8.float() - y16.float()).abs().max().item():.3e}"
    # and the staged grouped MLP outputs
    b8, b16 = d8.stage_buffers(), d16.stage_buffers()
    for d, b in ((d8, b8), (d16, b16)):
        d.route(b)
        d.permute(b)
        d.grouped_mlp(b)
    torch.cuda.synchronize()
    n = int(b8["offsets"][-1].item())
    assert torch.equal(b8["y_perm"][:n], b16["y_perm"][:n])
    if cfg.n_shared:
        assert torch.equal(b8["y_shared"], b16["y_shared"])
    P.say(f"  bit-identical over {n} routed rows")


def test_fp8_layer_is_deterministic_and_honours_the_stream():
    cfg = CASES[5]
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    ref = dev.forward().clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    dev.y.zero_()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(3):
            dev.forward(stream=s)
    s.synchronize()
    assert torch.equal(dev.y, ref)


def test_fp8_rejects_prefill_batches():
    from sparse_mixture_experts_29_amd import binding
    cfg = R(configs.mixtral_decode_fp8(64), d_model=256, d_ff=256)
    li = make_inputs(cfg)
    dev = DeviceLayer(li)
    big = cfg.replace(T=65)
    x = torch.zeros((65, cfg.d_model), dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty_like(x)
    ws = torch.empty(binding.moe_workspace_size(big, binding.MOE_OP_LAYER), dtype=torch.uint8, device="cuda:0")
    ex, sh = dev.fp8_experts()
    with pytest.raises(binding.MoeError) as e:
        binding.moe_layer_forward_fp8(big, x, dev.w_router, None, ex, sh, y, ws)
    assert e.value.status == binding.MOE_ERR_UNSUPPORTED
    assert np.isfinite(dev.forward().float().cpu().numpy()).all()
