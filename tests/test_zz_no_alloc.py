"""attn_decode_noalloc, the allocation-free entry point: the same kernels as
attn_decode with the split partials in the library's static per-GPU scratch.
Called through the C ABI and compared with attn_decode bit for bit (outputs
and stored cache entries), on two calls in a row, the second smaller; a call
past the scratch is rejected before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import bit_dequant_gemv_amd as bdg
import synth
from bit_dequant_gemv_amd import _lib
from tests.helpers import banner

pytestmark = pytest.mark.gpu


def _caches(cfg, layer, pos0, cap, dev):
    kv, vv, kb, vb = synth.attn_cache(cfg, layer, pos0, cap)
    kc = torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
    vc = torch.from_numpy(vb.view(np.int16)).to(dev).view(torch.bfloat16)
    return kc, vc


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def test_noalloc_equals_attn_decode_on_two_calls(dev):
    cfg = synth.ATTN["gptoss20b_attn_8k"]
    lib = _lib.load()
    cap = 4100
    table, _, _ = bdg.attn_rope_table(cfg.rope, cfg.head_dim, cap, device=dev)
    sinks = torch.from_numpy(synth.attn_sinks(cfg, 1)).to(dev)
    # first call: 4 tokens over 4000 cached keys (32 splits per token and KV
    # head, 4.3 MB of partials); second: 1 token in a 128-key window
    for step, (pos0, m, window) in enumerate(((4000, 4, 0), (700, 1, 128))):
        banner(f"attn_decode_noalloc call {step}: pos0={pos0} m={m} window={window}")
        q, k, v = (torch.from_numpy(a).to(dev) for a in synth.attn_token(cfg, 1, step, m))
        kc_a, vc_a = _caches(cfg, 1, pos0, cap, dev)
        kc_b, vc_b = kc_a.clone(), vc_a.clone()
        o_ref = bdg.attn_decode(q, k, v, kc_a, vc_a, pos0, table, cfg.sm_scale, sinks, window)
        o = torch.full_like(o_ref, float("nan"))
        st = lib.attn_decode_noalloc(_p(q), _p(k), _p(v), _p(kc_b), _p(vc_b), _lib.BDG_BF16, cap, cfg.n_heads,
                                     cfg.n_kv_heads, cfg.head_dim, m, pos0, _p(table), table.shape[0],
                                     cfg.sm_scale, _p(sinks), window, _p(o), _p(None))
        assert st == _lib.BDG_OK, lib.bdg_strerror(st)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {step}: outputs differ"
        assert torch.equal(kc_b.view(torch.int16), kc_a.view(torch.int16)), f"call {step}: stored keys differ"
        assert torch.equal(vc_b.view(torch.int16), vc_a.view(torch.int16)), f"call {step}: stored values differ"
        assert torch.all(torch.isfinite(o))


def test_noalloc_rejects_a_call_past_the_scratch(dev):
    cfg = synth.ATTN["gptoss20b_attn_8k"]
    lib = _lib.load()
    m, pos0, cap = 8, 100, 200            # 8 tokens x 8 KV heads: 8.65 MB of partials > 8 MiB
    need = lib.attn_decode_workspace(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, m, pos0 + m)
    assert need > _lib.BDG_ATTN_SCRATCH_BYTES
    table, _, _ = bdg.attn_rope_table(cfg.rope, cfg.head_dim, cap, device=dev)
    q, k, v = (torch.from_numpy(a).to(dev) for a in synth.attn_token(cfg, 1, 0, m))
    kc, vc = _caches(cfg, 1, pos0, cap, dev)
    o = torch.full((m, cfg.n_heads, cfg.head_dim), 3.0, device=dev)
    banner("attn_decode_noalloc past the scratch")
    st = lib.attn_decode_noalloc(_p(q), _p(k), _p(v), _p(kc), _p(vc), _lib.BDG_BF16, cap, cfg.n_heads,
                                 cfg.n_kv_heads, cfg.head_dim, m, pos0, _p(table), cap, cfg.sm_scale, None, 0,
                                 _p(o), None)
    assert st == _lib.BDG_E_TOO_LARGE
    assert b"scratch" in lib.bdg_strerror(st)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0), "a rejected call wrote its output"
