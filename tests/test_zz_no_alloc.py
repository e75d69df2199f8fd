"""moe_route_noalloc: moe_route with its scratch in a fixed device array (one per GPU) instead of
a caller's workspace, for callers that cannot allocate.  Its outputs must equal moe_route's bit for
bit on every call, including a call that follows a larger one on the same array (the array keeps
the previous call's contents), and a shape beyond the array must be refused before any launch."""
from __future__ import annotations

import ctypes
import math

import pytest
import torch

import mixture_experts_layer_adjusted_amd as moe
import synth
from mixture_experts_layer_adjusted_amd import binding
from synth.device import fill_normal_

pytestmark = pytest.mark.gpu


def _inputs(T, d, N, dtype, cid):
    u = torch.empty((T, d), dtype=torch.bfloat16 if dtype == moe.MOE_DTYPE_BF16 else torch.float32, device="cuda")
    fill_normal_(u, synth.stream_key(0, cid, synth.TAG_U, 0), 1.0)
    e = fill_normal_(torch.empty((N, d), dtype=torch.float32, device="cuda"),
                     synth.stream_key(0, cid, synth.TAG_CENTROID, 0), 1.0 / math.sqrt(d))
    b = fill_normal_(torch.empty((N,), dtype=torch.float32, device="cuda"), synth.stream_key(0, cid, synth.TAG_BIAS, 0),
                     0.1)
    return u, e, b


def _outputs(T, N, K, fill):
    return (torch.full((T, K), fill, dtype=torch.int32, device="cuda"),
            torch.full((T, K), float(fill), dtype=torch.float32, device="cuda"),
            torch.full((N,), fill, dtype=torch.int32, device="cuda"))


def _compare(T, d, N, K, dtype, cid):
    print(f"moe_route_noalloc vs moe_route: T={T} d={d} N_r={N} K_r={K} dtype={dtype}", flush=True)
    shape = moe.make_shape(T, d, N, K, 1, 128, dtype)
    u, e, b = _inputs(T, d, N, dtype, cid)
    ws = torch.empty(max(moe.moe_workspace_size(shape), 1), dtype=torch.uint8, device="cuda")
    ref = _outputs(T, N, K, -1)
    moe.moe_route(shape, u, e, b, *ref, ws)
    got = _outputs(T, N, K, -2)
    moe.moe_route_noalloc(shape, u, e, b, *got)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r.view(torch.int32), g.view(torch.int32))


def test_noalloc_route_matches_moe_route_on_consecutive_calls():
    # V3 prefill then a smaller V3 decode batch (split-K logits) on the same array, then the
    # VALU routers (bf16 with d not a multiple of 64, fp32), then no tokens at all
    _compare(16384, 7168, 256, 8, moe.MOE_DTYPE_BF16, 3)
    _compare(256, 7168, 256, 8, moe.MOE_DTYPE_BF16, 2)
    _compare(300, 200, 16, 4, moe.MOE_DTYPE_BF16, 91)
    _compare(77, 96, 12, 3, moe.MOE_DTYPE_F32, 92)
    shape = moe.make_shape(0, 128, 16, 4, 1, 64, moe.MOE_DTYPE_BF16)
    load = torch.full((16,), 5, dtype=torch.int32, device="cuda")
    moe.moe_route_noalloc(shape, None, None, None, None, None, load)
    torch.cuda.synchronize()
    assert torch.count_nonzero(load) == 0


def test_noalloc_route_refuses_shapes_beyond_its_array():
    lib = binding.raw_lib()
    # T = 65536 at the V3 shape needs more than the 64 MiB array (its affinities alone are 64 MiB)
    shape = moe.make_shape(65536, 7168, 256, 8, 1, 2048, moe.MOE_DTYPE_BF16)
    load = torch.full((256,), 7, dtype=torch.int32, device="cuda")
    fake = ctypes.c_void_p(0x1000)
    rc = lib.moe_route_noalloc(ctypes.byref(shape), fake, fake, fake, fake, fake, ctypes.c_void_p(load.data_ptr()),
                               None)
    assert rc == 3
    torch.cuda.synchronize()
    assert torch.all(load == 7)     # nothing was launched
