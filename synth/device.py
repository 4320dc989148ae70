"""Upload seeded synthetic workloads to the GPU and build decode plans.

Plumbing for tests and the benchmark: the arrays come from ``synth`` (host,
NumPy), torch holds them in device memory, and the plan is created through
the libbdg binding.  No arithmetic of the method happens here.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import synth
from bit_dequant_gemv_amd import MoEPlan, QWeight


def _t(arr, device):
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def qweight_from_arrays(fmt, arrays, group, device):
    """QWeight from (codes, scales[, zeros]) host arrays (2-D or expert-stacked 3-D)."""
    codes = _t(arrays[0], device)
    scales = _t(arrays[1], device)
    zeros = _t(arrays[2], device) if fmt == synth.FMT_INT4G else None
    return QWeight(fmt, codes, scales, zeros, group)


def upload_layer(cfg, layer, device, threads=8, experts=None):
    """Device tensors of one layer: router, bias, gate_up and down expert batches."""
    E = cfg.n_experts
    experts = range(E) if experts is None else experts
    w_r, b_r, hot = synth.router(cfg, layer)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda e: synth.expert_weights(cfg, layer, e), experts))
    n_arr = 3 if cfg.fmt == synth.FMT_INT4G else 2
    gu = [np.stack([p["gu"][i] for p in parts]) for i in range(n_arr)]
    dn = [np.stack([p["dn"][i] for p in parts]) for i in range(n_arr)]
    del parts
    return dict(
        w_router=_t(w_r, device),
        b_router=_t(b_r, device) if b_r is not None else None,
        hot=hot,
        gate_up=qweight_from_arrays(cfg.fmt, gu, cfg.group, device),
        down=qweight_from_arrays(cfg.fmt, dn, cfg.group, device),
    )


def build_plan(cfg, device, n_layers=None, max_m=None, use_graph=True, threads=8, layers=None, **plan_opts):
    """(plan, layer tensors) for the first n_layers layers of cfg; plan_opts
    go to MoEPlan (route_every_layer, per_token)."""
    n_layers = cfg.n_layers if n_layers is None else n_layers
    if layers is None:
        layers = [upload_layer(cfg, l, device, threads) for l in range(n_layers)]
    plan = MoEPlan(layers, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, fmt=cfg.fmt,
                   group=cfg.group, stack=cfg.norm, norm_eps=1e-5,
                   max_m=max_m if max_m is not None else cfg.m, use_graph=use_graph, **plan_opts)
    return plan, layers


def hidden_device(cfg, tokens, device):
    """Hidden states of the given tokens as a device tensor (bf16 or fp32) and host fp32 values."""
    vals, bits = synth.hidden_batch(cfg, tokens)
    if bits is not None:
        t = torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        t = torch.from_numpy(vals).to(device)
    return t, vals
