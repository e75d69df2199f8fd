"""moe_prepare_weights on the GPU: FP8_B128 packs the E4M3 codes and 128x128 block scales of every
stack (核心概念, FP8 item of the page "DeepSeek-V3 技術報告"), equal to the oracle's quantiser bit for
bit, and a forward on the prepared weights equals one on weights quantised stack by stack; BF16
hands the logical weights through."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_adjusted_amd as moe
from oracle import moe_oracle as O
from synth import bf16_bits_to_f32, host
from synth.configs import LayerConfig
from synth.device import host_to_device

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from helpers import Runner, quantize_fp8_weights

NAMES = ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")


def _logical(dev, cfg):
    ns = cfg.n_shared > 0
    return moe.make_weights(dev["w_gate"], dev["w_up"], dev["w_down"], dev["sh_gate"] if ns else None,
                            dev["sh_up"] if ns else None, dev["sh_down"] if ns else None)


@pytest.mark.parametrize("n_shared", [1, 0])
def test_prepare_fp8_weights(n_shared):
    cfg = LayerConfig(95 + n_shared, "prepare-fp8", 200, 256, 16, 4, n_shared, 384, "fp8", "uniform0.01")
    print(f"prepare: T={cfg.tokens} d={cfg.hidden} N={cfg.n_routed} Ns={cfg.n_shared} I={cfg.inter}", flush=True)
    h = host.make_host_inputs(cfg)
    dev = host_to_device(h)
    shape = moe.make_shape(cfg.tokens, cfg.hidden, cfg.n_routed, cfg.top_k, cfg.n_shared, cfg.inter,
                           moe.MOE_DTYPE_FP8_B128)
    logical = _logical(dev, cfg)
    nbytes = moe.moe_prepare_weights(shape, logical, size_only=True)
    packed = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    prepared = moe.moe_prepare_weights(shape, logical, packed)
    torch.cuda.synchronize()
    base = packed.data_ptr()
    pk = packed.cpu().numpy()
    for i, name in enumerate(NAMES):
        w = h[name]
        n, r, c = w.shape
        cptr, sptr = getattr(prepared, name), getattr(prepared, name + "_scale")
        if n == 0:
            assert cptr is None and sptr is None
            continue
        codes = pk[cptr - base: cptr - base + n * r * c].reshape(n, r, c)
        sc = pk[sptr - base: sptr - base + n * (r // 128) * (c // 128) * 4].view(np.float32).reshape(
            n, r // 128, c // 128)
        for e in range(n):
            c_o, s_o = O.quantize_weight_128x128(bf16_bits_to_f32(w[e]))
            assert np.array_equal(codes[e], c_o), (name, e)
            assert np.array_equal(sc[e].view(np.uint32), s_o.view(np.uint32)), (name, e)
    # a forward on the prepared weights equals one on the stack-by-stack quantised weights
    r = Runner(cfg, quantize_fp8_weights(dev, cfg))
    r.route()
    r.forward()
    out = torch.empty_like(r.out)
    moe.moe_forward(shape, dev["u"], prepared, r.idx, r.gate, out, r.ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), r.out.view(torch.int16))


def test_prepare_bf16_weights_pass_through():
    cfg = LayerConfig(97, "prepare-bf16", 64, 256, 16, 4, 1, 128, "bf16", "uniform0.01")
    dev = host_to_device(host.make_host_inputs(cfg))
    shape = moe.make_shape(cfg.tokens, cfg.hidden, cfg.n_routed, cfg.top_k, cfg.n_shared, cfg.inter,
                           moe.MOE_DTYPE_BF16)
    logical = _logical(dev, cfg)
    assert moe.moe_prepare_weights(shape, logical, size_only=True) == 0
    prepared = moe.moe_prepare_weights(shape, logical)
    for name in NAMES:
        assert getattr(prepared, name) == dev[name].data_ptr()
        assert getattr(prepared, name + "_scale") is None
