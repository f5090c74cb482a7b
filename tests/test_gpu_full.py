"""GPU parity at the full sizes of the five named workloads, in the launch configuration
the benchmark times: routing and permutation bit-exact on every token, and every row of the
expert outputs (y_perm), the shared-expert outputs and the layer output y compared with the
oracle element by element.
"""
import gc

import pytest
import torch

from sparse_mixture_experts_29_amd import configs
from sparse_mixture_experts_29_amd.device import DeviceLayer
from sparse_mixture_experts_29_amd.inputs import make_inputs
from tests import _parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    gc.collect()
    torch.cuda.empty_cache()


def test_tiny_fp32_full():
    cfg = configs.TINY_FP32
    P.say(f"case {cfg.name}")
    li = make_inputs(cfg)
    P.check_layer_full(li, DeviceLayer(li))


@pytest.mark.timeout(900)
def test_mixtral_decode_sweep_full():
    """T in {1, 4, 16, 64} tokens per step, the same weights, every row checked."""
    base = None
    for T in configs.DECODE_TS:
        cfg = configs.mixtral_decode(T)
        P.say(f"case {cfg.name}")
        li = make_inputs(cfg)
        dev = DeviceLayer(li, threads=16, weights_from=base)
        base = base or dev
        P.check_layer_full(li, dev)


@pytest.mark.timeout(900)
def test_mixtral_decode_fp8_sweep_full():
    """FP8 expert weights, T in {1, 4, 16, 64}: the same codes and scales, every row checked."""
    base = None
    for T in configs.DECODE_TS:
        cfg = configs.mixtral_decode_fp8(T)
        P.say(f"case {cfg.name}")
        li = make_inputs(cfg)
        dev = DeviceLayer(li, threads=16, weights_from=base)
        base = base or dev
        P.check_layer_full(li, dev)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [configs.MIXTRAL_PREFILL, configs.QWEN3_FINE, configs.QWEN3_FINE_CF,
                                 configs.DEEPSEEK_V3], ids=lambda c: c.name)
def test_prefill_layers_full(cfg):
    P.say(f"case {cfg.name}: generating {cfg.total_weight_bytes() / 1e9:.2f} GB of weights")
    li = make_inputs(cfg)
    dev = DeviceLayer(li, threads=16)
    P.say("  inputs resident")
    P.check_layer_full(li, dev)
