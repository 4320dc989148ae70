"""Seeded synthetic inputs for the MoE expert-decode workloads.

This module only draws random bytes and numbers; it holds none of the
method's arithmetic (no decoding, no products, no routing).  Both the oracle
(CPU) and the HIP path (GPU) are fed from it, so each side can regenerate any
tensor from its key alone.

Every tensor comes from its own PCG64 stream keyed by
SeedSequence([base, layer, expert, kind]); hidden states use
SeedSequence([base, 0xFFFF, token, 0]).  Expert codes are uniform bytes (both
nibbles uniform over all 16 codes); MXFP4 scale bytes are uniform integers in
[exp_lo, exp_hi]; int4 zero points are uniform nibbles and int4 scales are
U(scale_lo, scale_hi) rounded to fp16; router weights are N(0, sigma^2) fp32;
hidden states are N(0, 1), rounded to bf16 where the workload says so.

The workload shapes follow the pages: gpt-oss-20B experts are 2880 x 2880
with 32 experts, top-4, 24 layers; 120B has the same expert shape with 128
experts and 36 layers ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon",
section 3 Results, 120B viability microbench).  The 30B-class packed-int4 MoE
keeps about 15.4 GB resident ("Single-stream int4 decode of a 30B MoE on
Apple Silicon", section 1).
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor kinds (the last SeedSequence word)
K_GU_CODES, K_GU_SCALES, K_GU_ZEROS = 0, 1, 2
K_DN_CODES, K_DN_SCALES, K_DN_ZEROS = 3, 4, 5
K_ROUTER_W, K_ROUTER_B = 6, 7
HIDDEN_KEY = 0xFFFF

FMT_MXFP4 = "mxfp4"
FMT_INT4G = "int4g"


@dataclass(frozen=True)
class MoEConfig:
    name: str
    base: int            # seed base
    fmt: str             # "mxfp4" or "int4g"
    n_layers: int
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    group: int = 32      # 32 for MXFP4 (fixed by the format); int4 group size
    exp_lo: int = 118    # MXFP4 E8M0 exponent range, inclusive
    exp_hi: int = 128
    scale_lo: float = 0.005   # int4 fp16 scale range
    scale_hi: float = 0.02
    router_sigma: float = 0.02
    x_dtype: str = "bf16"     # hidden-state dtype handed to the path
    norm: bool = True         # RMSNorm + residual between layers (stacks)
    hot_experts: int = 0      # skewed routing: size of the hot set
    hot_bias: float = 0.0     # logit bias added to the hot set
    n_tokens: int = 64        # decode tokens (rows of M per step times steps)
    m: int = 1                # tokens per decode step
    extra: dict = field(default_factory=dict)


def _cfg(**kw):
    return MoEConfig(**kw)


# The five workloads.  "gemv" is the single-matrix microbench (treated as one
# layer of one expert whose gate_up is unused).
CONFIGS = {
    "gemv_2880": _cfg(name="gemv_2880", base=101, fmt=FMT_MXFP4, n_layers=1,
                      hidden=2880, inter=2880, n_experts=1, top_k=1,
                      exp_lo=120, exp_hi=130, x_dtype="f32", norm=False,
                      n_tokens=1),
    "gptoss20b_layer": _cfg(name="gptoss20b_layer", base=201, fmt=FMT_MXFP4,
                            n_layers=1, hidden=2880, inter=2880, n_experts=32,
                            top_k=4, norm=False, n_tokens=64),
    "gptoss20b_stack": _cfg(name="gptoss20b_stack", base=301, fmt=FMT_MXFP4,
                            n_layers=24, hidden=2880, inter=2880, n_experts=32,
                            top_k=4, n_tokens=64),
    "q4_30b_stack": _cfg(name="q4_30b_stack", base=401, fmt=FMT_INT4G,
                         n_layers=48, hidden=2048, inter=768, n_experts=128,
                         top_k=8, group=64, n_tokens=64),
    "gptoss120b_smallm": _cfg(name="gptoss120b_smallm", base=501, fmt=FMT_MXFP4,
                              n_layers=36, hidden=2880, inter=2880,
                              n_experts=128, top_k=4, hot_experts=8,
                              hot_bias=1.57, n_tokens=16 * 16, m=16),
}


@dataclass(frozen=True)
class DenseConfig:
    """A single packed weight matrix [n][k] applied to one token's input."""
    name: str
    base: int
    fmt: str
    n: int                    # rows (outputs)
    k: int                    # reduction length
    group: int = 32
    exp_lo: int = 118
    exp_hi: int = 128
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    x_dtype: str = "bf16"
    rotate: int = 2           # distinct matrices called in turn (their bytes exceed every cache)
    m: int = 1                # tokens per call


# Dense packed-weight GEMVs on the non-expert shapes around the path: the
# gpt-oss vocabulary head (201,088 rows over the 2880-wide hidden state; the
# pages' 201088-way argmax, "Sovereign gpt-oss-20B (MXFP4) on Apple Silicon",
# section 1) and the packed-int4 head-width matrix the tracker's fused int4
# kernel is timed on (32768 x 2048, tracker entry D110).
DENSE = {
    "lmhead_201088": DenseConfig(name="lmhead_201088", base=601, fmt=FMT_MXFP4, n=201088, k=2880, rotate=2),
    "int4_32768x2048": DenseConfig(name="int4_32768x2048", base=701, fmt=FMT_INT4G, n=32768, k=2048,
                                   group=64, rotate=16),
    # large-M (prefill) product of one gpt-oss expert's gate_up (5760 x 2880
    # MXFP4) with 4096 tokens quantized to MXFP8, on the MX-scaled matrix cores
    "mx_prefill_5760x2880": DenseConfig(name="mx_prefill_5760x2880", base=801, fmt=FMT_MXFP4, n=5760, k=2880,
                                        rotate=1, m=4096),
}


# Large-M (prefill) evaluation of one bare gpt-oss-20B-shape MoE layer: all
# tokens of a 4096-token prompt routed at once, the experts as grouped GEMMs on
# the MX-scaled matrix cores.
PREFILL = {
    "gptoss20b_prefill": MoEConfig(name="gptoss20b_prefill", base=901, fmt=FMT_MXFP4, n_layers=1, hidden=2880,
                                   inter=2880, n_experts=32, top_k=4, norm=False, n_tokens=4096, m=4096),
}


# Decode attention of gpt-oss-20B (the model the gpt-oss page ports; its
# attention has learned per-head sinks, a 128-token sliding window and YaRN,
# sections 1 and 3).  The head counts, head size, rotary parameters and the
# alternation of sliding and full layers are the public gpt-oss-20B
# configuration, which the pages do not print: 64 query heads sharing 8 KV
# heads of 64 dimensions, YaRN base 150000 with factor 32 over an original
# 4096-token context (beta_fast 32, beta_slow 1), scores scaled by 1/8, even
# layers sliding.  The decode token sits at position ctx - 1 with ctx - 1
# earlier keys in the cache.
GPTOSS_ROPE = dict(theta=150000.0, factor=32.0, beta_fast=32.0, beta_slow=1.0, orig_ctx=4096, truncate=False)

K_ATT_KC, K_ATT_VC, K_ATT_SINK, K_ATT_TOKEN = 10, 11, 12, 13
ATT_TOKEN_KEY = 0x10000


@dataclass(frozen=True)
class AttnConfig:
    name: str
    base: int
    n_layers: int
    n_heads: int = 64
    n_kv_heads: int = 8
    head_dim: int = 64
    ctx: int = 8192               # keys a full layer's decode token attends (its position + 1)
    window: int = 128             # keys a sliding layer's token attends
    cache_dtype: str = "bf16"
    m: int = 1                    # tokens per step
    sm_scale: float = 0.125
    sink_sigma: float = 1.0
    n_tokens: int = 64            # decode steps timed
    rope: dict = field(default_factory=lambda: dict(GPTOSS_ROPE))

    def sliding(self, layer):
        return layer % 2 == 0


ATTN = {
    "gptoss20b_attn_8k": AttnConfig(name="gptoss20b_attn_8k", base=1001, n_layers=24, ctx=8192),
}


def attn_cache(cfg: AttnConfig, layer, n_pos, cap=None):
    """Earlier keys and values of one layer: N(0, 1) at positions < n_pos of
    caches [n_kv_heads][cap][head_dim] (cap defaults to n_pos), rounded to
    bf16 for a bf16 cache.  Positions >= n_pos hold NaN (never attended).
    Returns (k values fp32, v values fp32, k bits, v bits); bits are the
    uint16 bf16 patterns for a bf16 cache and None for fp32."""
    cap = n_pos if cap is None else cap
    out = []
    for kind in (K_ATT_KC, K_ATT_VC):
        x = np.full((cfg.n_kv_heads, cap, cfg.head_dim), np.nan, dtype=np.float32)
        x[:, :n_pos] = rng_for(cfg.base, layer, 0, kind).standard_normal(
            (cfg.n_kv_heads, n_pos, cfg.head_dim), dtype=np.float32)
        out.append(x)
    if cfg.cache_dtype == "bf16":
        kb, vb = bf16_bits_of(out[0]), bf16_bits_of(out[1])
        return bf16_to_f32(kb), bf16_to_f32(vb), kb, vb
    return out[0], out[1], None, None


def attn_sinks(cfg: AttnConfig, layer):
    return (rng_for(cfg.base, layer, 0, K_ATT_SINK).standard_normal(cfg.n_heads) * cfg.sink_sigma).astype(
        np.float32)


def attn_token(cfg: AttnConfig, layer, step, m=None):
    """q [m][n_heads][d], k and v [m][n_kv_heads][d]: fp32 N(0, 1) projections."""
    m = cfg.m if m is None else m
    r = rng_for(cfg.base, layer, ATT_TOKEN_KEY + step, K_ATT_TOKEN)
    q = r.standard_normal((m, cfg.n_heads, cfg.head_dim), dtype=np.float32)
    k = r.standard_normal((m, cfg.n_kv_heads, cfg.head_dim), dtype=np.float32)
    v = r.standard_normal((m, cfg.n_kv_heads, cfg.head_dim), dtype=np.float32)
    return q, k, v


def rng_for(base, layer, expert, kind):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([base, layer, expert, kind])))


def uniform_bytes(rng, shape):
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def mxfp4_matrix(base, layer, expert, codes_kind, scales_kind, n, k, exp_lo, exp_hi):
    """(codes uint8 [n][k/2], scales uint8 [n][k/32]) for one MXFP4 matrix."""
    if k % 32:
        raise ValueError("MXFP4 K must be a multiple of 32")
    codes = uniform_bytes(rng_for(base, layer, expert, codes_kind), (n, k // 2))
    scales = rng_for(base, layer, expert, scales_kind).integers(
        exp_lo, exp_hi + 1, size=(n, k // 32), dtype=np.uint8)
    return codes, scales


def fp16_bits_of(values_f32):
    """fp16 bit patterns (uint16) of fp32 values, round-to-nearest-even."""
    return np.asarray(values_f32, dtype=np.float32).astype(np.float16).view(np.uint16)


def int4g_matrix(base, layer, expert, kinds, n, k, group, scale_lo, scale_hi):
    """(codes uint8 [n][k/2], scales fp16 bits uint16 [n][k/group],
    zeros uint8 [n][ceil(k/group/2)]) for one group-quantized int4 matrix."""
    if k % group or group % 32:
        raise ValueError("int4: K must be a multiple of the group, the group of 32")
    codes_kind, scales_kind, zeros_kind = kinds
    groups = k // group
    codes = uniform_bytes(rng_for(base, layer, expert, codes_kind), (n, k // 2))
    s32 = rng_for(base, layer, expert, scales_kind).uniform(
        scale_lo, scale_hi, size=(n, groups)).astype(np.float32)
    zeros = uniform_bytes(rng_for(base, layer, expert, zeros_kind), (n, (groups + 1) // 2))
    if groups % 2:
        zeros[:, -1] &= 0x0F   # the unused high nibble of an odd group count
    return codes, fp16_bits_of(s32), zeros


def expert_weights(cfg: MoEConfig, layer, expert):
    """Packed weights of one expert: dict with 'gu' and 'dn' tuples.

    gate_up is [2*inter][hidden] (g rows then u rows), down is [hidden][inter].
    """
    if cfg.fmt == FMT_MXFP4:
        gu = mxfp4_matrix(cfg.base, layer, expert, K_GU_CODES, K_GU_SCALES,
                          2 * cfg.inter, cfg.hidden, cfg.exp_lo, cfg.exp_hi)
        dn = mxfp4_matrix(cfg.base, layer, expert, K_DN_CODES, K_DN_SCALES,
                          cfg.hidden, cfg.inter, cfg.exp_lo, cfg.exp_hi)
    else:
        gu = int4g_matrix(cfg.base, layer, expert, (K_GU_CODES, K_GU_SCALES, K_GU_ZEROS),
                          2 * cfg.inter, cfg.hidden, cfg.group, cfg.scale_lo, cfg.scale_hi)
        dn = int4g_matrix(cfg.base, layer, expert, (K_DN_CODES, K_DN_SCALES, K_DN_ZEROS),
                          cfg.hidden, cfg.inter, cfg.group, cfg.scale_lo, cfg.scale_hi)
    return {"gu": gu, "dn": dn}


def gemv_matrix(cfg: MoEConfig, index=0):
    """The single GEMV microbench matrix number ``index`` ([hidden][hidden] MXFP4)."""
    return mxfp4_matrix(cfg.base, index, 0, K_DN_CODES, K_DN_SCALES,
                        cfg.hidden, cfg.hidden, cfg.exp_lo, cfg.exp_hi)


def dense_matrix(cfg: DenseConfig, index=0):
    """Packed arrays of dense matrix number ``index`` (see DENSE)."""
    if cfg.fmt == FMT_MXFP4:
        return mxfp4_matrix(cfg.base, index, 0, K_DN_CODES, K_DN_SCALES, cfg.n, cfg.k, cfg.exp_lo, cfg.exp_hi)
    return int4g_matrix(cfg.base, index, 0, (K_DN_CODES, K_DN_SCALES, K_DN_ZEROS), cfg.n, cfg.k, cfg.group,
                        cfg.scale_lo, cfg.scale_hi)


def router(cfg: MoEConfig, layer):
    """(W_r fp32 [E][H], bias fp32 [E] or None, hot set or None) for one layer.

    With a hot set, the bias is +hot_bias on ``hot_experts`` experts drawn
    per layer, 0 elsewhere.
    """
    w = (rng_for(cfg.base, layer, 0, K_ROUTER_W).standard_normal(
        (cfg.n_experts, cfg.hidden)) * cfg.router_sigma).astype(np.float32)
    if cfg.hot_experts <= 0:
        return w, None, None
    rng = rng_for(cfg.base, layer, 0, K_ROUTER_B)
    hot = np.sort(rng.choice(cfg.n_experts, size=cfg.hot_experts, replace=False))
    bias = np.zeros(cfg.n_experts, dtype=np.float32)
    bias[hot] = np.float32(cfg.hot_bias)
    return w, bias, hot


def bf16_bits_of(values_f32):
    """bf16 bit patterns (uint16) of fp32 values, round-to-nearest-even."""
    u = np.ascontiguousarray(values_f32, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)          # no overflow below the all-ones NaN patterns
    r += u
    r += np.uint32(0x7FFF)
    r >>= 16
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def hidden(cfg, token, n=None):
    """Hidden state of one token, N(0, 1) (length hidden, or k for a dense
    matrix).

    Returns (values as fp32, bits): bits is the bf16 uint16 array for bf16
    workloads (values are then exactly bf16) and None for fp32 ones.
    """
    if n is None:
        n = cfg.k if isinstance(cfg, DenseConfig) else cfg.hidden
    x = rng_for(cfg.base, HIDDEN_KEY, token, 0).standard_normal(n).astype(np.float32)
    if cfg.x_dtype == "bf16":
        bits = bf16_bits_of(x)
        return bf16_to_f32(bits), bits
    return x, None


def hidden_batch(cfg: MoEConfig, tokens):
    vals, bits = zip(*(hidden(cfg, t) for t in tokens))
    vals = np.stack(vals)
    return vals, (None if bits[0] is None else np.stack(bits))


def random_input(seed, shape, kind="normal", lo=0, hi=255):
    """Generic seeded arrays for small parity cases."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xABCD])))
    if kind == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    if kind == "bytes":
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    if kind == "int":
        return rng.integers(lo, hi + 1, size=shape, dtype=np.int64)
    raise ValueError(kind)
