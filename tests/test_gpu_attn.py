"""GPU parity of the decode attention (attn_rope_table, attn_decode) against
oracle/attn.py.

Bars: the rotary table, the YaRN inverse frequencies and the attention
scaling are fp32 roundings of float64 values, equal to the oracle's bit for
bit (an entry may differ only where the float64 value sits within a few
float64 ulps of a rounding midpoint, which is checked); cache entries the call
stores are bit-exact; outputs agree with the float64 oracle within
``attn.output_bound`` per (token, head) and within 2e-5 of the largest value
magnitude in the window (the fp32 arithmetic lands far inside the worst-case
bound; a dropped or doubled key moves an output by about 1/n of a value).
"""

import numpy as np
import pytest
import torch

import bit_dequant_gemv_amd as bdg
import synth
from oracle import attn
from tests.helpers import banner

pytestmark = pytest.mark.gpu

GPTOSS = synth.GPTOSS_ROPE
OUT_ABS = 2e-5            # |o - o_ref| <= OUT_ABS * max |v| of the window


def _assert_rounding_of(got32, want64, what):
    got32 = np.asarray(got32, dtype=np.float32)
    want32 = np.asarray(want64, dtype=np.float64).astype(np.float32)
    bad = np.nonzero(got32.view(np.uint32) != want32.view(np.uint32))[0] if got32.ndim == 1 else \
        np.argwhere(got32.view(np.uint32) != want32.view(np.uint32))
    if len(bad) == 0:
        return
    # only a float64 value within a few float64 ulps of an fp32 midpoint may round either way
    g = got32[tuple(bad.T)] if got32.ndim > 1 else got32[bad]
    w = np.asarray(want64)[tuple(bad.T)] if got32.ndim > 1 else np.asarray(want64)[bad]
    half_ulp = np.spacing(np.abs(g).astype(np.float32)).astype(np.float64) / 2
    near = np.abs(np.abs(g.astype(np.float64) - w) - half_ulp) <= 8 * np.spacing(np.abs(w))
    assert near.all(), f"{what}: {len(bad)} entries are not a rounding of the float64 value, e.g. {bad[:3]}"


@pytest.mark.parametrize("params,d,n_pos", [
    (dict(GPTOSS), 64, 131072),
    (dict(GPTOSS, truncate=True), 64, 4096),
    (dict(theta=10000.0, factor=8.0, beta_fast=32.0, beta_slow=1.0, orig_ctx=2048, truncate=False), 128, 2048),
    (dict(theta=500000.0, factor=1.0, beta_fast=32.0, beta_slow=1.0, orig_ctx=8192, truncate=False), 64, 1000),
], ids=["gptoss", "gptoss_truncate", "d128_s8", "plain"])
def test_rope_table_matches_oracle(dev, params, d, n_pos):
    banner(f"rope table {params} d={d} n_pos={n_pos}")
    tab, inv, scale = bdg.attn_rope_table(params, d, n_pos, device=dev)
    torch.cuda.synchronize()
    inv64, a64 = attn.yarn_inv_freq(d, params["theta"], params["factor"], params["orig_ctx"],
                                    params["beta_fast"], params["beta_slow"], params["truncate"])
    _assert_rounding_of(inv.cpu().numpy(), inv64, "inv_freq")
    _assert_rounding_of(scale.cpu().numpy(), np.array([a64]), "attn_scale")
    inv32, a32 = inv.cpu().numpy(), scale.cpu().numpy()[0]
    assert np.array_equal(inv32, inv64.astype(np.float32)) and a32 == np.float32(a64)
    # every row from the oracle's float64 phasor (same fp32 constants)
    f = inv32.astype(np.float64)
    pos = np.arange(n_pos, dtype=np.float64)[:, None]
    ang = pos * f[None, :]
    want = np.concatenate([np.cos(ang) * float(a32), np.sin(ang) * float(a32)], axis=1)
    _assert_rounding_of(tab.cpu().numpy(), want, "table")


def _upload_cache(kb, kv, dtype, dev):
    if dtype == "bf16":
        return torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(kv).to(dev)


def _cache_values(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def _cache_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def _run_case(dev, cfg, layer, pos0, m, window, with_sinks, workspace=None, table=None):
    cap = pos0 + m + 3
    kv, vv, kb, vb = synth.attn_cache(cfg, layer, pos0, cap)
    q, k, v = synth.attn_token(cfg, layer, 0, m)
    sinks = synth.attn_sinks(cfg, layer) if with_sinks else None
    kc = _upload_cache(kb, kv, cfg.cache_dtype, dev)
    vc = _upload_cache(vb, vv, cfg.cache_dtype, dev)
    kc0, vc0 = _cache_bits(kc), _cache_bits(vc)
    if table is None:
        table, _, _ = bdg.attn_rope_table(cfg.rope, cfg.head_dim, cap, device=dev)
    qd, kd, vd = (torch.from_numpy(a).to(dev) for a in (q, k, v))
    sd = torch.from_numpy(sinks).to(dev) if with_sinks else None
    o = bdg.attn_decode(qd, kd, vd, kc, vc, pos0, table, cfg.sm_scale, sd, window, workspace=workspace)
    torch.cuda.synchronize()
    inv32, a32 = attn.rope_constants(cfg.head_dim, **{k_: cfg.rope[k_] for k_ in
                                                      ("theta", "factor", "orig_ctx", "beta_fast", "beta_slow",
                                                       "truncate")})
    # the oracle's cache: earlier entries as stored, later ones never read
    o_ref, kc_ref, vc_ref = attn.decode_step(q, k, v, np.nan_to_num(kv.astype(np.float64)),
                                             np.nan_to_num(vv.astype(np.float64)), cfg.cache_dtype, pos0, inv32,
                                             a32, window, cfg.sm_scale, sinks)
    # stored entries bit-exact, everything else untouched
    kc1, vc1 = _cache_bits(kc), _cache_bits(vc)
    new = slice(pos0, pos0 + m)
    assert np.array_equal(np.delete(kc1, np.s_[pos0:pos0 + m], axis=1), np.delete(kc0, np.s_[pos0:pos0 + m], axis=1))
    assert np.array_equal(np.delete(vc1, np.s_[pos0:pos0 + m], axis=1), np.delete(vc0, np.s_[pos0:pos0 + m], axis=1))
    assert np.array_equal(_cache_values(kc)[:, new], kc_ref[:, new]), "stored keys differ"
    assert np.array_equal(_cache_values(vc)[:, new], vc_ref[:, new]), "stored values differ"
    # outputs
    pos = pos0 + np.arange(m)
    q_rot = attn.rotate64(q, np.broadcast_to(pos[:, None], q.shape[:2]), inv32, a32)
    bound = attn.output_bound(q_rot, kc_ref, vc_ref, pos, window, cfg.sm_scale)
    got = o.cpu().numpy().astype(np.float64)
    err = np.abs(got - o_ref).max(axis=2)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"max err {err.max():.3e} above bound at {np.argwhere(err > bound)[:3]}"
    group = cfg.n_heads // cfg.n_kv_heads
    for t in range(m):
        lo = max(0, pos[t] - window + 1) if window else 0
        vmax = np.abs(vc_ref[:, lo:pos[t] + 1]).max(axis=(1, 2))           # per kv head
        assert np.all(err[t] <= OUT_ABS * np.repeat(vmax, group)), f"token {t}: err {err[t].max():.3e}"
    return err.max()


CASES = [
    # (cache dtype, pos0, m, window, sinks, kv heads)
    ("bf16", 0, 1, 0, True, 8),          # first token, empty cache
    ("bf16", 37, 1, 0, True, 2),         # one block
    ("bf16", 300, 1, 0, True, 2),        # three blocks, ragged last
    ("f32", 300, 1, 0, False, 2),
    ("bf16", 300, 1, 128, True, 2),      # sliding window, one block
    ("bf16", 1000, 5, 128, True, 2),     # five tokens, each its own window
    ("bf16", 250, 7, 0, True, 1),        # new keys across a block boundary
    ("f32", 500, 16, 5, True, 2),        # tiny window
    ("bf16", 127, 2, 0, True, 8),        # second token's own key alone in its block
    ("bf16", 4000, 1, 0, True, 8),       # 32 blocks
    ("f32", 4000, 3, 0, False, 8),       # 32 splits
    ("f32", 5000, 2, 0, True, 2),        # two sub-chunks per block (running maximum rescaled)
    ("bf16", 10000, 1, 0, True, 1),      # two sub-chunks per block
    ("bf16", 20000, 3, 300, True, 2),    # long cache, window of 300
    ("bf16", 65536, 1, 0, True, 1),      # 64K keys: eight sub-chunks per block
    ("f32", 30000, 2, 0, True, 1),       # fp32 cache, several sub-chunks per block
    ("bf16", 3000, 64, 0, True, 1),      # the largest chunk: 64 tokens, up to 64 own keys each
    ("bf16", 200, 64, 40, True, 2),      # 64 tokens, windows mostly inside the chunk itself
]


@pytest.mark.parametrize("dtype,pos0,m,window,sinks,hkv", CASES,
                         ids=[f"{c[0]}-p{c[1]}-m{c[2]}-w{c[3]}-{'s' if c[4] else 'ns'}-kv{c[5]}" for c in CASES])
def test_attention_cases(dev, dtype, pos0, m, window, sinks, hkv):
    cfg = synth.AttnConfig(name="case", base=1101 + pos0 + m, n_layers=1, n_kv_heads=hkv, n_heads=8 * hkv,
                           cache_dtype=dtype, sink_sigma=2.0)
    banner(f"attn case dtype={dtype} pos0={pos0} m={m} window={window} sinks={sinks} hkv={hkv}")
    _run_case(dev, cfg, 0, pos0, m, window, sinks)


def test_workspace_reuse_across_calls(dev):
    # one workspace for calls of different sizes, holding the previous call's partials
    cfg = synth.AttnConfig(name="reuse", base=1201, n_layers=1, n_kv_heads=4, n_heads=32)
    ws = bdg.attn_workspace(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, 4, 3000, dev)
    for pos0, m in ((2900, 4), (700, 1), (2000, 3), (129, 2)):
        banner(f"attn reuse pos0={pos0} m={m}")
        _run_case(dev, cfg, 0, pos0, m, 0, True, workspace=ws)



@pytest.mark.parametrize("layer", [0, 1], ids=["sliding", "full"])
def test_gptoss20b_8k_layer(dev, layer):
    # the benchmark's launch: 64 query heads, 8 KV heads, bf16 cache, the
    # decode token at position 8191
    cfg = synth.ATTN["gptoss20b_attn_8k"]
    window = cfg.window if cfg.sliding(layer) else 0
    banner(f"attn gpt-oss-20B layer {layer} window={window} ctx={cfg.ctx}")
    ws = bdg.attn_workspace(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, 1, cfg.ctx, dev)
    _run_case(dev, cfg, layer, cfg.ctx - 1, 1, window, True, workspace=ws)


def test_repeat_calls_are_deterministic(dev):
    cfg = synth.ATTN["gptoss20b_attn_8k"]
    kv, vv, kb, vb = synth.attn_cache(cfg, 1, 3000, 3001)
    q, k, v = synth.attn_token(cfg, 1, 0)
    table, _, _ = bdg.attn_rope_table(cfg.rope, 64, 3001, device=dev)
    kc = _upload_cache(kb, kv, "bf16", dev)
    vc = _upload_cache(vb, vv, "bf16", dev)
    ws = bdg.attn_workspace(64, 8, 64, 1, 3001, dev)
    qd, kd, vd = (torch.from_numpy(a).to(dev) for a in (q, k, v))
    sd = torch.from_numpy(synth.attn_sinks(cfg, 1)).to(dev)
    outs = [bdg.attn_decode(qd, kd, vd, kc, vc, 3000, table, 0.125, sd, 0, workspace=ws).clone() for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_bad_arguments(dev):
    cfg = synth.ATTN["gptoss20b_attn_8k"]
    table, _, _ = bdg.attn_rope_table(cfg.rope, 64, 16, device=dev)
    q = torch.zeros(1, 64, 64, device=dev)
    k = torch.zeros(1, 8, 64, device=dev)
    kc = torch.zeros(8, 16, 64, device=dev, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError):                      # past the cache
        bdg.attn_decode(q, k, k, kc, kc.clone(), 16, table, 0.125)
    with pytest.raises(ValueError):                        # unsupported head grouping
        bdg.attn_decode(torch.zeros(1, 32, 64, device=dev), k, k, kc, kc.clone(), 3, table, 0.125)
    with pytest.raises(ValueError):
        bdg.attn_decode(q, k, k, kc.half(), kc.half(), 3, table, 0.125)
