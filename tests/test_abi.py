"""The C ABI without a GPU: header compiles as C and C++, the struct layout agrees with
the binding, the library exports every declared symbol, and host-side validation and
size queries behave as documented (none of these calls touches the device)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from sparse_mixture_experts_29_amd import binding, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

lib_built = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH), reason="libmoe.so not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(binding.EXPORTS)


@pytest.mark.parametrize("compiler,lang", [("gcc", "c"), ("g++", "c++")])
def test_header_compiles_standalone(tmp_path, compiler, lang):
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "moe.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   "int main(void){ printf(\"%zu %zu %zu %zu %zu\\n\", sizeof(moe_config),"
                   " offsetof(moe_config, capacity_factor), offsetof(moe_config, n_shared),"
                   " offsetof(moe_config, dtype), offsetof(moe_config, reserved)); return 0; }\n")
    exe = tmp_path / "t"
    subprocess.run([compiler, "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    C = binding.MoeConfig
    assert [int(v) for v in out] == [ctypes.sizeof(C), C.capacity_factor.offset, C.n_shared.offset,
                                     C.dtype.offset, C.reserved.offset]


@lib_built
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(declared_functions()) <= exported
    # internal symbols stay hidden
    assert not [s for s in re.findall(r"\bT (\S+)", out) if "launch_" in s]
    lib = binding.load_library()
    for name in declared_functions():
        assert getattr(lib, name) is not None


@lib_built
def test_status_strings():
    for s in range(5):
        assert binding.status_string(s).startswith("MOE_")
    assert "unknown" in binding.status_string(99)


def _cfg(**kw):
    base = dict(T=100, d_model=128, d_ff=256, n_experts=8, top_k=2, gating=0, capacity_factor=0.0,
                n_shared=0, d_ff_shared=0, dtype=1, reserved=0)
    base.update(kw)
    return binding.MoeConfig(**base)


@lib_built
@pytest.mark.parametrize("kw,status", [
    ({}, binding.MOE_OK),
    (dict(top_k=0), binding.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), binding.MOE_ERR_INVALID_ARG),
    (dict(n_experts=0), binding.MOE_ERR_INVALID_ARG),
    (dict(T=-1), binding.MOE_ERR_INVALID_ARG),
    (dict(gating=2), binding.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), binding.MOE_ERR_INVALID_ARG),
    (dict(n_shared=1, d_ff_shared=0), binding.MOE_ERR_INVALID_ARG),
    (dict(reserved=1), binding.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=float("inf")), binding.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=float("nan")), binding.MOE_ERR_INVALID_ARG),
    (dict(d_model=100), binding.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=96), binding.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=2048, top_k=2), binding.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=64, top_k=33), binding.MOE_ERR_UNSUPPORTED),
    # activation matrices of 4 GiB and more (32-bit row offsets in the tiled GEMMs)
    (dict(T=1 << 20, d_model=2048, d_ff=256), binding.MOE_ERR_UNSUPPORTED),
    (dict(T=(1 << 19) - 1, d_model=4096, d_ff=256), binding.MOE_OK),
    (dict(T=1 << 18, d_model=256, d_ff=4096, top_k=2), binding.MOE_ERR_UNSUPPORTED),
    (dict(T=0), binding.MOE_OK),
])
def test_config_validation(kw, status):
    assert binding.moe_check_config(_cfg(**kw)) == status


@lib_built
def test_null_config_and_null_out_params():
    lib = binding.load_library()
    assert lib.moe_check_config(None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_size(ctypes.byref(_cfg()), 0, None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_size(ctypes.byref(_cfg()), 9, ctypes.byref(ctypes.c_size_t())) == \
        binding.MOE_ERR_INVALID_ARG


@lib_built
def test_entry_points_reject_bad_arguments_before_touching_the_device():
    lib = binding.load_library()
    c = ctypes.byref(_cfg())
    assert lib.moe_route(c, None, None, None, None, None, None, None) == binding.MOE_ERR_INVALID_ARG
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    assert lib.moe_permute(c, fake, fake, fake, fake, fake, fake, fake, 0, None) == binding.MOE_ERR_WORKSPACE
    assert lib.moe_layer_forward(c, fake, fake, None, fake, fake, fake, None, None, None, fake, fake, 16,
                                 None) == binding.MOE_ERR_WORKSPACE
    cs = ctypes.byref(_cfg(n_shared=1, d_ff_shared=128))
    assert lib.moe_grouped_mlp(cs, fake, fake, fake, fake, fake, fake, None, None, None, fake, None, fake,
                               1 << 40, None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(cs, fake, fake, fake, None, fake, None) == binding.MOE_ERR_INVALID_ARG
    # T = 0 is a no-op, even with NULL buffers
    c0 = ctypes.byref(_cfg(T=0))
    assert lib.moe_layer_forward(c0, None, None, None, None, None, None, None, None, None, None, None, 0,
                                 None) == binding.MOE_OK


@lib_built
def test_expert_shard_rejects_bad_arguments_before_touching_the_device():
    lib = binding.load_library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    args = (fake, fake, fake, fake, fake, fake, fake)
    ok = _cfg(top_k=1)
    # a shard runs top-1 rows, dropless, without shared experts
    for bad in (_cfg(top_k=2), _cfg(top_k=1, capacity_factor=1.25), _cfg(top_k=1, n_shared=1, d_ff_shared=128)):
        assert lib.moe_expert_shard_forward(ctypes.byref(bad), *args, 1 << 40, None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_shard_forward(ctypes.byref(ok), fake, None, fake, fake, fake, fake, fake, 1 << 40,
                                        None) == binding.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_shard_forward(ctypes.byref(ok), *args, 16, None) == binding.MOE_ERR_WORKSPACE
    assert lib.moe_expert_shard_forward(ctypes.byref(_cfg(T=0, top_k=1)), None, None, None, None, None, None,
                                        None, 0, None) == binding.MOE_OK


@lib_built
@pytest.mark.parametrize("cfg", list(configs.ALL.values()), ids=lambda c: c.name)
def test_capacity_and_max_kept_match_the_oracle(cfg):
    C = oracle.expert_capacity(cfg.capacity_factor, cfg.T, cfg.top_k, cfg.n_experts)
    assert binding.moe_capacity(cfg) == (-1 if C is None else C)
    pairs = cfg.T * cfg.top_k
    assert binding.moe_max_kept(cfg) == (pairs if C is None else min(pairs, C * cfg.n_experts))
    for op in (binding.MOE_OP_PERMUTE, binding.MOE_OP_GROUPED_MLP, binding.MOE_OP_LAYER):
        assert binding.moe_workspace_size(cfg, op) % 256 == 0


@lib_built
@pytest.mark.parametrize("cf,T,k,E", [(1.25, 8192, 8, 128), (0.3, 1000, 3, 7), (1.1, 777, 2, 8),
                                      (2.0 / 3.0, 999, 5, 13), (0.01, 12, 1, 2)])
def test_capacity_rounding_agrees_with_the_oracle(cf, T, k, E):
    c = _cfg(T=T, top_k=k, n_experts=E, capacity_factor=cf)
    assert binding.moe_capacity(c) == oracle.expert_capacity(cf, T, k, E)


def test_fp8_weights_struct_layout(tmp_path):
    src = tmp_path / "f.c"
    src.write_text('#include "moe.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   "int main(void){ printf(\"%zu %zu %zu\\n\", sizeof(moe_fp8_weights),"
                   " offsetof(moe_fp8_weights, w_down), offsetof(moe_fp8_weights, scale_down)); return 0; }\n")
    exe = tmp_path / "f"
    subprocess.run(["gcc", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", str(src), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    W = binding.MoeFp8Weights
    assert out == [ctypes.sizeof(W), W.w_down.offset, W.scale_down.offset]


def _fp8(base=0x1000, **kw):
    """A moe_fp8_weights of fake, 16-byte aligned device addresses (never dereferenced)."""
    f = dict(w_gate=base, w_up=base + 0x100, w_down=base + 0x200, scale_gate=base + 0x300,
             scale_up=base + 0x400, scale_down=base + 0x500)
    f.update(kw)
    return binding.MoeFp8Weights(**f)


@lib_built
def test_fp8_entry_points_reject_bad_arguments_before_touching_the_device():
    lib = binding.load_library()
    fake = ctypes.c_void_p(0x1000)
    ex = ctypes.byref(_fp8())
    big = 1 << 40

    def layer(cfg, experts=ex, shared=None, ws_bytes=big):
        return lib.moe_layer_forward_fp8(ctypes.byref(cfg), fake, fake, None, experts, shared, fake, fake, ws_bytes,
                                         None)

    def grouped(cfg, experts=ex, shared=None, y_shared=None, ws_bytes=big):
        return lib.moe_grouped_mlp_fp8(ctypes.byref(cfg), fake, fake, fake, experts, shared, fake, y_shared, fake,
                                       ws_bytes, None)

    small = _cfg(T=64)
    # FP8 weights run on the weight-streaming path only: bf16 activations, at most 64 tokens
    assert layer(_cfg(T=65)) == binding.MOE_ERR_UNSUPPORTED
    assert grouped(_cfg(T=4096)) == binding.MOE_ERR_UNSUPPORTED
    assert layer(_cfg(T=4, dtype=binding.MOE_F32)) == binding.MOE_ERR_UNSUPPORTED
    # every member present and 16-byte aligned
    assert layer(small, experts=None) == binding.MOE_ERR_INVALID_ARG
    assert layer(small, experts=ctypes.byref(_fp8(scale_up=None))) == binding.MOE_ERR_INVALID_ARG
    assert layer(small, experts=ctypes.byref(_fp8(w_down=0x1008))) == binding.MOE_ERR_INVALID_ARG
    assert grouped(small, experts=ctypes.byref(_fp8(scale_gate=0x1004))) == binding.MOE_ERR_INVALID_ARG
    # the shared struct (and y_shared) are required with shared experts, ignored without
    sh_cfg = _cfg(T=8, n_shared=1, d_ff_shared=128)
    assert layer(sh_cfg) == binding.MOE_ERR_INVALID_ARG
    assert grouped(sh_cfg, shared=ex) == binding.MOE_ERR_INVALID_ARG  # no y_shared
    assert layer(sh_cfg, shared=ctypes.byref(_fp8(w_up=None))) == binding.MOE_ERR_INVALID_ARG
    assert layer(small, shared=ctypes.byref(_fp8(w_up=None)), ws_bytes=16) == binding.MOE_ERR_WORKSPACE
    assert grouped(small, ws_bytes=16) == binding.MOE_ERR_WORKSPACE
    # T = 0 is a no-op
    assert lib.moe_layer_forward_fp8(ctypes.byref(_cfg(T=0)), None, None, None, None, None, None, None, 0,
                                     None) == binding.MOE_OK


@lib_built
def test_fp8_workspace_is_the_dtype_layer_workspace():
    for cfg in (configs.mixtral_decode_fp8(t) for t in configs.DECODE_TS):
        dt = cfg.replace(weights="dtype")
        for op in (binding.MOE_OP_GROUPED_MLP, binding.MOE_OP_LAYER):
            assert binding.moe_workspace_size(cfg, op) == binding.moe_workspace_size(dt, op)


def test_layer_grads_struct_layout(tmp_path):
    src = tmp_path / "g.c"
    src.write_text('#include "moe.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   "int main(void){ printf(\"%zu %zu %zu\\n\", sizeof(moe_layer_grads),"
                   " offsetof(moe_layer_grads, dw_down), offsetof(moe_layer_grads, aux_loss)); return 0; }\n")
    exe = tmp_path / "g"
    subprocess.run(["gcc", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", str(src), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    G = binding.MoeLayerGrads
    assert out == [ctypes.sizeof(G), G.dw_down.offset, G.aux_loss.offset]


@lib_built
def test_backward_rejects_bad_arguments_before_touching_the_device():
    lib = binding.load_library()
    fake = ctypes.c_void_p(0x1000)
    g = binding.MoeLayerGrads(*([0x2000] * 10))

    def bwd(cfg, grads=g, dy=fake, aux=0.0, ws_bytes=1 << 40, shared=(None, None, None)):
        return lib.moe_layer_backward(ctypes.byref(cfg), fake, fake, None, fake, fake, fake, *shared, dy, aux,
                                      ctypes.byref(grads) if grads is not None else None, fake, ws_bytes, None)

    assert bwd(_cfg(dtype=binding.MOE_F32)) == binding.MOE_ERR_UNSUPPORTED
    assert bwd(_cfg(), aux=float("nan")) == binding.MOE_ERR_INVALID_ARG
    assert bwd(_cfg(), dy=None) == binding.MOE_ERR_INVALID_ARG
    assert bwd(_cfg(), grads=None) == binding.MOE_ERR_INVALID_ARG
    assert bwd(_cfg(), grads=binding.MoeLayerGrads(0x2000, None, *([0x2000] * 8))) == binding.MOE_ERR_INVALID_ARG
    sh = _cfg(n_shared=1, d_ff_shared=128)
    assert bwd(sh) == binding.MOE_ERR_INVALID_ARG  # no shared weights
    assert bwd(sh, shared=(fake, fake, fake),
               grads=binding.MoeLayerGrads(*([0x2000] * 6), None, None, None, None)) == binding.MOE_ERR_INVALID_ARG
    assert bwd(_cfg(), ws_bytes=16) == binding.MOE_ERR_WORKSPACE
    assert lib.moe_layer_backward(ctypes.byref(_cfg(T=0)), *([None] * 10), 0.0, None, None, 0, None) == binding.MOE_OK
    # the optional outputs may be NULL
    opt = binding.MoeLayerGrads(0x2000, 0x2000, None, 0x2000, 0x2000, 0x2000, None, None, None, None)
    assert bwd(_cfg(), grads=opt, ws_bytes=16) == binding.MOE_ERR_WORKSPACE


@lib_built
def test_backward_workspace_sizes():
    for cfg in (configs.MIXTRAL_PREFILL, configs.QWEN3_FINE, configs.DEEPSEEK_V3):
        b = binding.moe_workspace_size(cfg, binding.MOE_OP_LAYER_BACKWARD)
        assert b % 256 == 0
        # holds the recomputed x Wg | x Wu, u, da | db and h of every pair (12 f bytes a pair)
        assert b >= cfg.T * cfg.top_k * 12 * cfg.d_ff
    # and no copy of the expert weights: the dgrad launches read them as stored
    ds = configs.DEEPSEEK_V3
    assert binding.moe_workspace_size(ds, binding.MOE_OP_LAYER_BACKWARD) < ds.n_experts * 3 * ds.d_model * ds.d_ff * 2
    with pytest.raises(binding.MoeError):
        binding.moe_workspace_size(configs.TINY_FP32, binding.MOE_OP_LAYER_BACKWARD)
