"""The hot path captured once in a HIP graph (torch.cuda.CUDAGraph over the library's launches)
and replayed: every replay reproduces the eager results bit for bit, with eager calls that
change the routing in between.  The library launches kernels only (no allocation, memset, copy
or synchronisation on its stream), so a caller can capture moe_route + moe_forward +
moe_update_bias once and replay it per batch."""
from __future__ import annotations

import pytest
import torch

import mixture_experts_layer_adjusted_amd as moe
from synth import host
from synth.configs import CONFIGS, LayerConfig
from synth.device import host_to_device

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from helpers import Runner, quantize_fp8_weights


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", ["mid-bf16", "fp8-small"])
def test_graph_replay_matches_eager(name):
    cfg = CONFIGS[1] if name == "mid-bf16" else LayerConfig(76, "fp8-graph", 1000, 512, 32, 4, 1, 256, "fp8",
                                                            "normal_var0.01")
    print(f"graph replay: {cfg.name} T={cfg.tokens} d={cfg.hidden} N={cfg.n_routed} dtype={cfg.dtype}", flush=True)
    dev = host_to_device(host.make_host_inputs(cfg))
    if cfg.dtype == "fp8":
        dev = quantize_fp8_weights(dev, cfg)
    r = Runner(cfg, dev)
    T, K, N = cfg.tokens, cfg.top_k, cfg.n_routed
    bias0 = dev["bias"].clone()

    def step(bias):
        moe.moe_route(r.shape, dev["u"], dev["centroids"], bias, r.idx, r.gate, r.load, r.ws)
        moe.moe_forward(r.shape, dev["u"], r.weights, r.idx, r.gate, r.out, r.ws)
        moe.moe_update_bias(N, T * K, r.load, bias, cfg.gamma)

    b = bias0.clone()
    step(b)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (r.idx, r.gate, r.load, r.out, b)]

    gbias = bias0.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gbias)
    other = bias0 + 0.05 * torch.randn_like(bias0)
    for rep in range(3):
        gbias.copy_(bias0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (r.idx, r.gate, r.load, r.out, gbias)
        for k, (x, y) in enumerate(zip(got, ref)):
            assert torch.equal(_bits(x), _bits(y)), (rep, k)
        # eager work between replays that rewrites every output with another routing
        ob = other.clone()
        step(ob)
        torch.cuda.synchronize()
        assert not torch.equal(r.idx, ref[0])


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_training_step_graph_replay_matches_eager(dtype):
    """moe_route + moe_forward_train + moe_backward_saved captured once and replayed: the output,
    du, the centroid and weight gradients equal the eager step's bit for bit on every replay, with
    an eager step on another routing in between."""
    cfg = LayerConfig(88, f"train-graph-{dtype}", 512, 512, 16, 4, 1, 256, dtype, "normal_var0.01")
    print(f"training-step graph replay: {cfg.name} T={cfg.tokens} d={cfg.hidden} N={cfg.n_routed}", flush=True)
    dev = host_to_device(host.make_host_inputs(cfg))
    if dtype == "fp8":
        dev = quantize_fp8_weights(dev, cfg)
    r = Runner(cfg, dev)
    T, d, N = cfg.tokens, cfg.hidden, cfg.n_routed
    saved = torch.empty(moe.moe_saved_inputs_size(r.shape) // 2, dtype=torch.bfloat16, device="cuda")
    ws_b = torch.empty(moe.moe_backward_workspace_size(r.shape), dtype=torch.uint8, device="cuda")
    dout = (torch.randn((T, d), device="cuda") * 0.5).to(torch.bfloat16)
    du = torch.empty_like(dout)
    de = torch.empty((N, d), dtype=torch.float32, device="cuda")
    grads = {k: torch.empty(dev[k].shape, dtype=torch.bfloat16, device="cuda")
             for k in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")}
    wg = moe.make_weight_grads(*(grads[k] for k in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")))
    bias0 = dev["bias"].clone()

    def step(bias):
        moe.moe_route(r.shape, dev["u"], dev["centroids"], bias, r.idx, r.gate, r.load, r.ws)
        moe.moe_forward_train(r.shape, dev["u"], r.weights, r.idx, r.gate, r.out, saved, r.ws)
        moe.moe_backward_saved(r.shape, dev["u"], dev["centroids"], r.weights, r.idx, r.gate, saved, dout, du, de, wg,
                               ws_b)

    def outputs():
        return [r.idx, r.out, du, de] + [grads[k] for k in sorted(grads)]

    step(bias0)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(bias0)
    other = bias0 + 0.05 * torch.randn_like(bias0)
    for rep in range(3):
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (x, y) in enumerate(zip(outputs(), ref)):
            assert torch.equal(_bits(x), _bits(y)), (rep, k)
        step(other)
        torch.cuda.synchronize()
        assert not torch.equal(r.idx, ref[0])
