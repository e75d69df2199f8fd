"""Device-resident seeded inputs (torch tensors on a GPU), bit-identical to synth.host.

Small tensors (centroids, bias) are drawn on the host and copied; large ones
(tokens, expert weights) are drawn in place by the HIP filler.  bf16 tensors
have torch dtype bfloat16; the fp8 configuration's weights are drawn in bf16
(quantisation is a library step, not an input).
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from . import (TAG_SH_DOWN, TAG_SH_GATE, TAG_SH_UP, TAG_U, TAG_W_DOWN, TAG_W_GATE, TAG_W_UP, normal_scale32,
               stream_key)
from .configs import LayerConfig
from .host import bias_vector, centroids, storage_is_bf16
from .native import device_lib


def fill_normal_(t: torch.Tensor, key: int, sigma: float, start: int = 0) -> torch.Tensor:
    """Fill a contiguous fp32/bf16 device tensor with elements [start, start+numel) of a stream."""
    assert t.is_cuda and t.is_contiguous() and t.dtype in (torch.float32, torch.bfloat16)
    kind = 0 if t.dtype == torch.float32 else 1
    rc = device_lib().synth_fill_normal_device(ctypes.c_void_p(t.data_ptr()), t.numel(), start, key,
                                               float(normal_scale32(sigma)), kind,
                                               ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_device failed ({rc})")
    return t


def _stack(cfg, n, rows, cols, tag, sigma, dt, dev):
    w = torch.empty((n, rows, cols), dtype=dt, device=dev)
    for e in range(n):
        fill_normal_(w[e], stream_key(cfg.seed, cfg.cid, tag, e), sigma)
    return w


def make_device_inputs(cfg: LayerConfig, device="cuda") -> dict:
    dt = torch.bfloat16 if storage_is_bf16(cfg) else torch.float32
    d, I, N, Ns = cfg.hidden, cfg.inter, cfg.n_routed, cfg.n_shared
    out = {}
    out["u"] = fill_normal_(torch.empty((cfg.tokens, d), dtype=dt, device=device),
                            stream_key(cfg.seed, cfg.cid, TAG_U, 0), 1.0)
    out["centroids"] = torch.from_numpy(centroids(cfg)).to(device)
    out["bias"] = torch.from_numpy(bias_vector(cfg)).to(device)
    sd, si = 1.0 / math.sqrt(d), 1.0 / math.sqrt(I)
    out["w_gate"] = _stack(cfg, N, I, d, TAG_W_GATE, sd, dt, device)
    out["w_up"] = _stack(cfg, N, I, d, TAG_W_UP, sd, dt, device)
    out["w_down"] = _stack(cfg, N, d, I, TAG_W_DOWN, si, dt, device)
    out["sh_gate"] = _stack(cfg, Ns, I, d, TAG_SH_GATE, sd, dt, device)
    out["sh_up"] = _stack(cfg, Ns, I, d, TAG_SH_UP, sd, dt, device)
    out["sh_down"] = _stack(cfg, Ns, d, I, TAG_SH_DOWN, si, dt, device)
    return out


def host_to_device(arrs: dict, device="cuda") -> dict:
    """Upload synth.host arrays (bf16 as uint16 bits) as torch tensors of the right dtype."""
    out = {}
    for k, a in arrs.items():
        if a.dtype == np.uint16:
            out[k] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out


def bf16_to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
