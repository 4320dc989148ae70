"""Thin torch-facing wrappers over libbdg, one per C entry point, same names.

Torch supplies device memory and the current HIP stream; every step of the
computation runs in the HIP kernels of ``libbdg.so``.  Nothing here computes
on the CPU, and there is no fallback path.
"""

import ctypes

import torch

from . import _lib
from ._lib import (BDG_BF16, BDG_E_WAIT, BDG_F32, BDG_FMT_INT4G, BDG_FMT_MXFP4, BDG_MOE_NO_GRAPH,
                   BDG_MOE_PER_TOKEN, BDG_MOE_ROUTE_EVERY_LAYER, BDG_MOE_STACK, BDG_MOE_FUSED_LAYER, BDG_MOE_MFMA,
                   BDG_MOE_ROUTE_KERNEL, BDG_OK, BDG_ROUTER_RMSNORM, LayerDesc, MoEDesc, QMat, Rope, check)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, shape, name):
    """Raise ValueError unless tensor t has exactly this shape."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _x_dtype(x):
    if x.dtype == torch.float32:
        return BDG_F32
    if x.dtype == torch.bfloat16:
        return BDG_BF16
    raise ValueError("activations must be float32 or bfloat16")


class QWeight:
    """A packed matrix [n][k], or a batch of experts [E][n][k], in the PLAIN layout.

    MXFP4: codes uint8 [..., n, k/2], scales uint8 [..., n, k/32].
    INT4G: codes uint8 [..., n, k/2], scales int16 (fp16 bits) [..., n, k/group],
           zeros uint8 [..., n, ceil(k/group/2)].
    """

    def __init__(self, fmt, codes, scales, zeros=None, group=32):
        if fmt not in ("mxfp4", "int4g"):
            raise ValueError("fmt must be 'mxfp4' or 'int4g'")
        self.fmt = fmt
        self.codes, self.scales, self.zeros = codes, scales, zeros
        self.group = 32 if fmt == "mxfp4" else int(group)
        self.n = codes.shape[-2]
        self.k = 2 * codes.shape[-1]
        self.batched = codes.dim() == 3
        self.n_experts = codes.shape[0] if self.batched else 1
        if codes.dim() not in (2, 3):
            raise ValueError("codes must be [n][k/2] or [E][n][k/2]")
        lead = tuple(codes.shape[:-1])
        if self.k % 32 or self.k % self.group:
            raise ValueError("k must be a multiple of 32 and of the group size")
        _shape(scales, lead + (self.k // self.group,), "scales")
        if fmt == "int4g":
            _shape(zeros, lead + ((self.k // self.group + 1) // 2,), "zeros")
        _dev_ptr(codes, "codes", torch.uint8)
        _dev_ptr(scales, "scales", torch.uint8 if fmt == "mxfp4" else torch.int16)
        if fmt == "int4g":
            _dev_ptr(zeros, "zeros", torch.uint8)
        self.scale_words = None

    def stage_mx_scales(self):
        """Write the stage-major copy of the MXFP4 scales that the MX
        matrix-core products read (mx_stage_scales; once per matrix, again
        after the scales change); later qmat() views carry it."""
        if self.fmt != "mxfp4":
            raise ValueError("stage_mx_scales is for MXFP4 matrices")
        self.scale_words = None
        qm = self.qmat()
        lib = _lib.load()
        nbytes = lib.mx_scale_words_bytes(ctypes.byref(qm), self.n_experts)
        if nbytes < 0:
            raise ValueError("invalid matrix for mx_stage_scales")
        words = torch.empty(nbytes // 4, dtype=torch.int32, device=self.codes.device)
        check("mx_stage_scales", lib.mx_stage_scales(ctypes.byref(qm), self.n_experts,
                                                     _dev_ptr(words, "scale_words", torch.int32), nbytes, _stream()))
        self.scale_words = words
        return self

    def qmat(self):
        def stride(t):
            return t[0].numel() * t.element_size() if (t is not None and self.batched) else 0
        return QMat(
            fmt=BDG_FMT_MXFP4 if self.fmt == "mxfp4" else BDG_FMT_INT4G,
            group=self.group, n=self.n, k=self.k,
            codes=self.codes.data_ptr(), scales=self.scales.data_ptr(),
            zeros=self.zeros.data_ptr() if self.zeros is not None else None,
            expert_stride_codes=stride(self.codes), expert_stride_scales=stride(self.scales),
            expert_stride_zeros=stride(self.zeros),
            mx_scale_words=self.scale_words.data_ptr() if self.scale_words is not None else None)


def mxfp4_dequant(codes, scales, out_dtype=torch.float32):
    n, half_k = codes.shape
    _shape(scales, (n, 2 * half_k // 32), "scales")
    out = torch.empty((n, 2 * half_k), dtype=out_dtype, device=codes.device)
    odt = BDG_F32 if out_dtype == torch.float32 else BDG_BF16
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    check("mxfp4_dequant", _lib.load().mxfp4_dequant(
        _dev_ptr(codes, "codes", torch.uint8), _dev_ptr(scales, "scales", torch.uint8),
        n, 2 * half_k, _dev_ptr(out, "out"), odt, _stream()))
    return out


def int4g_dequant(codes, scales, zeros, group):
    n, half_k = codes.shape
    group = int(group)
    if group <= 0 or (2 * half_k) % group:
        raise ValueError("k must be a multiple of the group size")
    _shape(scales, (n, 2 * half_k // group), "scales")
    _shape(zeros, (n, (2 * half_k // group + 1) // 2), "zeros")
    out = torch.empty((n, 2 * half_k), dtype=torch.float32, device=codes.device)
    check("int4g_dequant", _lib.load().int4g_dequant(
        _dev_ptr(codes, "codes", torch.uint8), _dev_ptr(scales, "scales", torch.int16),
        _dev_ptr(zeros, "zeros", torch.uint8), n, 2 * half_k, int(group),
        _dev_ptr(out, "out"), _stream()))
    return out


def qgemv(w: QWeight, x, out=None):
    """y = W x for x [k] or [m][k]; returns fp32 [n] or [m][n]."""
    squeeze = x.dim() == 1
    x2 = x.reshape(1, -1) if squeeze else x
    m = x2.shape[0]
    if x2.shape[1] != w.k:
        raise ValueError("x and W disagree on K")
    if out is not None:
        _shape(out, (w.n,) if squeeze else (m, w.n), "out")
    y = out if out is not None else torch.empty((m, w.n), dtype=torch.float32, device=x.device)
    qm = w.qmat()
    check("qgemv", _lib.load().qgemv(ctypes.byref(qm), _dev_ptr(x2, "x"), _x_dtype(x2), m,
                                     _dev_ptr(y, "y", torch.float32), _stream()))
    return y[0] if squeeze and out is None else y


def mxfp8_quantize(x, codes=None, scales=None):
    """MXFP8 quantization of activations x [m][k] (fp32 or bf16): returns
    (codes uint8 [m][k], scales uint8 [m][k/32])."""
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    m, k = x2.shape
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    if codes is None:
        codes = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.uint8, device=x.device)
    _shape(codes, (m, k), "codes")
    _shape(scales, (m, k // 32), "scales")
    check("mxfp8_quantize", _lib.load().mxfp8_quantize(
        _dev_ptr(x2, "x"), _x_dtype(x2), m, k, _dev_ptr(codes, "codes", torch.uint8),
        _dev_ptr(scales, "scales", torch.uint8), _stream()))
    return codes, scales


def mx_gemm_workspace_bytes(n, k, m):
    nb = _lib.load().mx_gemm_workspace(n, k, m)
    if nb < 0:
        raise ValueError("invalid mx_gemm shape")
    return int(nb)


def mx_gemm(w: QWeight, codes, scales, out=None, workspace=None):
    """y [m][n] = W xq^T for MXFP4 W [n][k] and MXFP8 activations (codes [m][k],
    scales [m][k/32]) on the MX-scaled matrix cores.  workspace: a uint8
    device tensor of mx_gemm_workspace_bytes(n, k, m) bytes or more (made
    here when not given)."""
    m = codes.shape[0]
    if codes.dim() != 2 or codes.shape[1] != w.k or tuple(scales.shape) != (m, w.k // 32):
        raise ValueError("activation shapes do not match W")
    if out is not None:
        _shape(out, (m, w.n), "out")
    y = out if out is not None else torch.empty((m, w.n), dtype=torch.float32, device=codes.device)
    if workspace is None:
        workspace = torch.empty(mx_gemm_workspace_bytes(w.n, w.k, m), dtype=torch.uint8, device=codes.device)
    qm = w.qmat()
    check("mx_gemm", _lib.load().mx_gemm(ctypes.byref(qm), _dev_ptr(codes, "codes", torch.uint8),
                                         _dev_ptr(scales, "scales", torch.uint8), m,
                                         _dev_ptr(y, "y", torch.float32),
                                         _dev_ptr(workspace, "workspace", torch.uint8), workspace.numel(),
                                         _stream()))
    return y


def moe_prefill_mx(layer, n_experts, top_k, x, y=None, workspace=None):
    """One bare MoE layer over m tokens on the MX-scaled matrix cores.

    layer: dict with w_router [E][H] fp32, b_router or None, gate_up QWeight
    [E][2I][H] and down QWeight [E][H][I] (MXFP4).  Returns (y [m][H] fp32,
    idx [m][k] int32, w [m][k] fp32).  ``workspace`` (a uint8 device tensor of
    at least ``prefill_workspace_bytes`` bytes) is allocated when not given.
    """
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    m, hid = x2.shape
    gu, dn = layer["gate_up"], layer["down"]
    inter = dn.k
    if gu.k != hid or gu.n != 2 * inter or dn.n != hid:
        raise ValueError("gate_up must be [E][2I][H] and down [E][H][I] for x [m][H]")
    if gu.n_experts != n_experts or dn.n_experts != n_experts:
        raise ValueError("expert batches must hold n_experts matrices")
    _shape(layer["w_router"], (n_experts, hid), "w_router")
    _shape(layer.get("b_router"), (n_experts,), "b_router")
    if y is not None:
        _shape(y, (m, hid), "y")
    need = prefill_workspace_bytes(m, hid, inter, n_experts, top_k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    if y is None:
        y = torch.empty((m, hid), dtype=torch.float32, device=x.device)
    idx = torch.empty((m, top_k), dtype=torch.int32, device=x.device)
    wts = torch.empty((m, top_k), dtype=torch.float32, device=x.device)
    desc = LayerDesc()
    desc.w_router = _dev_ptr(layer["w_router"], "w_router", torch.float32).value
    b = layer.get("b_router")
    desc.b_router = _dev_ptr(b, "b_router", torch.float32).value if b is not None else None
    desc.gate_up = gu.qmat()
    desc.down = dn.qmat()
    check("moe_prefill_mx", _lib.load().moe_prefill_mx(
        ctypes.byref(desc), n_experts, top_k, _dev_ptr(x2, "x"), _x_dtype(x2), m,
        _dev_ptr(y, "y", torch.float32), _dev_ptr(idx, "idx", torch.int32), _dev_ptr(wts, "wts", torch.float32),
        _dev_ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream()))
    return y, idx, wts


def prefill_workspace_views(workspace, m, hidden, inter, n_experts, top_k):
    """Views of the parts of a moe_prefill_mx workspace (the layout include/bdg.h
    states: 256-byte aligned parts in order), plus "hq_scales": h's scale
    bytes as [P][I/32], arranged (a copy) from its stage-major words.  For
    inspection only."""
    P = m * top_k
    sh, si = (hidden // 32 + 3) // 4, (inter // 32 + 3) // 4
    sizes = [("xq", m * hidden, torch.uint8, (m, hidden)),
             ("xq_scales", m * (hidden // 32), torch.uint8, (m, hidden // 32)),
             ("row_off", 4 * (n_experts + 1), torch.int32, (n_experts + 1,)),
             ("tile_off", 4 * (n_experts + 1), torch.int32, (n_experts + 1,)),
             ("row_src", 4 * P, torch.int32, (P,)),
             ("pick_row", 4 * P, torch.int32, (P,)),
             ("hq", P * inter, torch.uint8, (P, inter)),
             ("xq_scale_words", 4 * sh * P, torch.uint8, (sh, P, 4)),
             ("hq_scale_words", 4 * si * P, torch.uint8, (si, P, 4)),
             ("gate_up_scale_words", 4 * sh * 2 * inter * n_experts, torch.uint8, (n_experts, sh, 2 * inter, 4)),
             ("down_scale_words", 4 * si * hidden * n_experts, torch.uint8, (n_experts, si, hidden, 4)),
             ("d", 4 * P * hidden, torch.float32, (P, hidden))]
    out, off = {}, 0
    for name, nbytes, dt, shape in sizes:
        out[name] = workspace[off:off + nbytes].view(dt).view(shape)
        off += (nbytes + 255) // 256 * 256
    out["hq_scales"] = out["hq_scale_words"].permute(1, 0, 2).reshape(P, 4 * si)[:, :inter // 32]
    return out


def prefill_workspace_bytes(m, hidden, inter, n_experts, top_k):
    n = _lib.load().moe_prefill_mx_workspace(m, hidden, inter, n_experts, top_k)
    if n < 0:
        raise ValueError("invalid prefill shape")
    return int(n)


def _rope(rope):
    r = Rope()
    r.theta, r.factor = float(rope["theta"]), float(rope["factor"])
    r.beta_fast, r.beta_slow = float(rope["beta_fast"]), float(rope["beta_slow"])
    r.orig_ctx, r.truncate = int(rope["orig_ctx"]), int(bool(rope.get("truncate", False)))
    return r


def attn_rope_table(rope, head_dim, n_pos, device=None, table=None):
    """Rotary table [n_pos][head_dim] fp32 for YaRN parameters ``rope`` (a dict
    with theta, factor, beta_fast, beta_slow, orig_ctx, truncate).  Returns
    (table, inv_freq [head_dim/2], attn_scale [1]), all device tensors."""
    device = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    if table is None:
        table = torch.empty((n_pos, head_dim), dtype=torch.float32, device=device)
    inv = torch.empty(head_dim // 2, dtype=torch.float32, device=device)
    scale = torch.empty(1, dtype=torch.float32, device=device)
    r = _rope(rope)
    check("attn_rope_table", _lib.load().attn_rope_table(
        ctypes.byref(r), head_dim, n_pos, _dev_ptr(table, "table", torch.float32),
        _dev_ptr(inv, "inv_freq", torch.float32), _dev_ptr(scale, "attn_scale", torch.float32), _stream()))
    return table, inv, scale


def attn_decode_workspace_bytes(n_heads, n_kv_heads, head_dim, m, max_keys):
    n = _lib.load().attn_decode_workspace(n_heads, n_kv_heads, head_dim, m, max_keys)
    if n < 0:
        raise ValueError("attention shape not supported")
    return int(n)


def attn_workspace(n_heads, n_kv_heads, head_dim, m, max_keys, device):
    """A workspace for attn_decode calls of up to m tokens."""
    n = attn_decode_workspace_bytes(n_heads, n_kv_heads, head_dim, m, max_keys)
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_decode(q, k, v, k_cache, v_cache, pos0, table, sm_scale, sinks=None, window=0, o=None,
                workspace=None):
    """One attention step of m new tokens (positions pos0 .. pos0 + m - 1).

    q [m][Hq][64], k and v [m][Hkv][64] fp32; caches [Hkv][cap][64] bf16 or
    fp32 (updated in place with the new rotated keys and values); table from
    attn_rope_table; sinks [Hq] fp32 or None; window 0 = full attention.
    Returns o [m][Hq][64] fp32.  A workspace is allocated when not given
    (reuse one across calls with attn_workspace)."""
    m, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (m, hkv, d) or v.shape != (m, hkv, d):
        raise ValueError("k and v must be [m][n_kv_heads][head_dim]")
    if k_cache.dtype != v_cache.dtype or k_cache.shape != v_cache.shape or k_cache.shape[0] != hkv:
        raise ValueError("caches must match and be [n_kv_heads][cap][head_dim]")
    cdt = {torch.bfloat16: BDG_BF16, torch.float32: BDG_F32}.get(k_cache.dtype)
    if cdt is None:
        raise ValueError("caches must be bfloat16 or float32")
    if q.dim() != 3 or k_cache.dim() != 3 or k_cache.shape[2] != d:
        raise ValueError("q must be [m][n_heads][head_dim] and caches [n_kv_heads][cap][head_dim]")
    if table.dim() != 2 or table.shape[1] != d:
        raise ValueError("table must be [positions][head_dim]")
    _shape(sinks, (hq,), "sinks")
    _shape(o, (m, hq, d), "o")
    cap = k_cache.shape[1]
    last = pos0 + m
    max_keys = min(window, last) if window > 0 else last
    need = attn_decode_workspace_bytes(hq, hkv, d, m, max_keys)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    if o is None:
        o = torch.empty((m, hq, d), dtype=torch.float32, device=q.device)
    check("attn_decode", _lib.load().attn_decode(
        _dev_ptr(q, "q", torch.float32), _dev_ptr(k, "k", torch.float32), _dev_ptr(v, "v", torch.float32),
        _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), cdt, cap, hq, hkv, d, m, pos0,
        _dev_ptr(table, "table", torch.float32), table.shape[0], float(sm_scale),
        _dev_ptr(sinks, "sinks", torch.float32), int(window), _dev_ptr(o, "o", torch.float32),
        _dev_ptr(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream()))
    return o


def attn_decode_noalloc(q, k, v, k_cache, v_cache, pos0, table, sm_scale, sinks=None, window=0, o=None):
    """attn_decode without a workspace: the library's static scratch holds the
    split partials (for callers that cannot allocate device memory; calls
    that overlap in time on one GPU race).  Returns o [m][Hq][64] fp32 (pass
    o to keep the call allocation-free on the torch side too)."""
    m, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (m, hkv, d) or v.shape != (m, hkv, d):
        raise ValueError("k and v must be [m][n_kv_heads][head_dim]")
    if k_cache.dtype != v_cache.dtype or k_cache.shape != v_cache.shape or k_cache.shape[0] != hkv:
        raise ValueError("caches must match and be [n_kv_heads][cap][head_dim]")
    if k_cache.dim() != 3 or k_cache.shape[2] != d or table.dim() != 2 or table.shape[1] != d:
        raise ValueError("caches must be [n_kv_heads][cap][head_dim] and table [positions][head_dim]")
    cdt = {torch.bfloat16: BDG_BF16, torch.float32: BDG_F32}.get(k_cache.dtype)
    if cdt is None:
        raise ValueError("caches must be bfloat16 or float32")
    _shape(sinks, (hq,), "sinks")
    if o is None:
        o = torch.empty((m, hq, d), dtype=torch.float32, device=q.device)
    _shape(o, (m, hq, d), "o")
    check("attn_decode_noalloc", _lib.load().attn_decode_noalloc(
        _dev_ptr(q, "q", torch.float32), _dev_ptr(k, "k", torch.float32), _dev_ptr(v, "v", torch.float32),
        _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), cdt, k_cache.shape[1], hq, hkv, d, m, pos0,
        _dev_ptr(table, "table", torch.float32), table.shape[0], float(sm_scale),
        _dev_ptr(sinks, "sinks", torch.float32), int(window), _dev_ptr(o, "o", torch.float32), _stream()))
    return o


def moe_router_topk(x, w_r, b_r=None, topk=4, rmsnorm=False, eps=1e-5):
    """(idx [m][k] int32, wts [m][k] fp32, logits [m][E] fp32)."""
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    m, h = x2.shape
    e = w_r.shape[0]
    _shape(w_r, (e, h), "w_r")
    _shape(b_r, (e,), "b_r")
    if not 1 <= topk <= e:
        raise ValueError("need 1 <= topk <= number of experts")
    idx = torch.empty((m, topk), dtype=torch.int32, device=x.device)
    wts = torch.empty((m, topk), dtype=torch.float32, device=x.device)
    logits = torch.empty((m, e), dtype=torch.float32, device=x.device)
    check("moe_router_topk", _lib.load().moe_router_topk(
        _dev_ptr(x2, "x"), _x_dtype(x2), _dev_ptr(w_r, "w_r", torch.float32),
        _dev_ptr(b_r, "b_r", torch.float32), m, h, e, topk,
        BDG_ROUTER_RMSNORM if rmsnorm else 0, float(eps),
        _dev_ptr(idx, "idx"), _dev_ptr(wts, "wts"), _dev_ptr(logits, "logits"), _stream()))
    return idx, wts, logits


class MoEPlan:
    """A decode plan (moe_plan_create) over per-layer device weights.

    layers: list of dicts with keys w_router [E][H] fp32, b_router [E] fp32 or
    None, gate_up QWeight [E][2I][H], down QWeight [E][H][I].  The plan keeps
    references to every tensor it points at.
    """

    def __init__(self, layers, hidden, inter, n_experts, top_k, fmt="mxfp4", group=32,
                 stack=True, norm_eps=1e-5, max_m=1, use_graph=True, route_every_layer=False,
                 per_token=False, fused_layer=False, mfma=False, route_kernel=False, wait_polls=0):
        self._layers = layers
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.n_layers = len(layers)
        self.stack = stack
        self.max_m = max_m
        arr = (LayerDesc * len(layers))()
        for i, L in enumerate(layers):
            gu, dn = L["gate_up"], L["down"]
            if gu.n != 2 * inter or gu.k != hidden or dn.n != hidden or dn.k != inter:
                raise ValueError(f"layer {i}: gate_up must be [E][2I][H] and down [E][H][I]")
            if gu.n_experts != n_experts or dn.n_experts != n_experts:
                raise ValueError(f"layer {i}: expert batches must hold n_experts matrices")
            _shape(L["w_router"], (n_experts, hidden), f"layer {i} w_router")
            _shape(L.get("b_router"), (n_experts,), f"layer {i} b_router")
            arr[i].w_router = _dev_ptr(L["w_router"], "w_router", torch.float32).value
            b = L.get("b_router")
            arr[i].b_router = _dev_ptr(b, "b_router", torch.float32).value if b is not None else None
            arr[i].gate_up = L["gate_up"].qmat()
            arr[i].down = L["down"].qmat()
        flags = ((BDG_MOE_STACK if stack else 0) | (0 if use_graph else BDG_MOE_NO_GRAPH)
                 | (BDG_MOE_ROUTE_EVERY_LAYER if route_every_layer else 0)
                 | (BDG_MOE_PER_TOKEN if per_token else 0)
                 | (BDG_MOE_FUSED_LAYER if fused_layer else 0)
                 | (BDG_MOE_MFMA if mfma else 0)
                 | (BDG_MOE_ROUTE_KERNEL if route_kernel else 0))
        desc = MoEDesc(n_layers=len(layers), hidden=hidden, inter=inter, n_experts=n_experts,
                       top_k=top_k, fmt=BDG_FMT_MXFP4 if fmt == "mxfp4" else BDG_FMT_INT4G,
                       group=32 if fmt == "mxfp4" else group, flags=flags,
                       norm_eps=norm_eps, max_m=max_m, layers=arr, wait_polls=int(wait_polls))
        handle = ctypes.c_void_p()
        check("moe_plan_create", _lib.load().moe_plan_create(ctypes.byref(desc), ctypes.byref(handle)))
        self._handle = handle
        self._desc_layers = arr

    @property
    def handle(self):
        if self._handle is None:
            raise RuntimeError("plan is closed")
        return self._handle

    def check(self):
        """moe_plan_check: True if no in-kernel wait gave up since the last
        check (False: some step's outputs were made NaN).  Synchronous."""
        st = _lib.load().moe_plan_check(self.handle, _stream())
        if st == BDG_E_WAIT:
            return False
        check("moe_plan_check", st)
        return True

    def close(self):
        if getattr(self, "_handle", None) is not None:
            _lib.load().moe_plan_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_expert_decode(plan: MoEPlan, x, y=None, traces=False):
    """One decode step of x [m][H]; returns y [m][H] fp32 (and traces if asked).

    traces=True also returns dict(topk [L][m][k] int32, wts [L][m][k] fp32,
    resid [L][m][H] fp32), the per-layer routing and input residual.
    """
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    m = x2.shape[0]
    _shape(x2, (m, plan.hidden), "x")
    if not 1 <= m <= plan.max_m:
        raise ValueError(f"m must be in [1, {plan.max_m}] (the plan's max_m)")
    if y is None:
        y = torch.empty((m, plan.hidden), dtype=torch.float32, device=x.device)
    _shape(y, (m, plan.hidden), "y")
    tr = None
    if traces:
        L, k, H = plan.n_layers, plan.top_k, plan.hidden
        tr = dict(topk=torch.empty((L, m, k), dtype=torch.int32, device=x.device),
                  wts=torch.empty((L, m, k), dtype=torch.float32, device=x.device),
                  resid=torch.empty((L, m, H), dtype=torch.float32, device=x.device))
    check("moe_expert_decode", _lib.load().moe_expert_decode(
        plan.handle, _dev_ptr(x2, "x"), _x_dtype(x2), m, _dev_ptr(y, "y", torch.float32),
        _dev_ptr(tr["topk"], "topk") if tr else None,
        _dev_ptr(tr["wts"], "wts") if tr else None,
        _dev_ptr(tr["resid"], "resid") if tr else None, _stream()))
    return (y, tr) if traces else y


def moe_experts_routed(plan: MoEPlan, layer, x, idx, wts, y=None):
    """Experts of one layer with fixed routing: y[t] = sum_j wts[t][j] FFN_{idx[t][j]}(x[t])."""
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    m = x2.shape[0]
    _shape(x2, (m, plan.hidden), "x")
    if not 1 <= m <= plan.max_m:
        raise ValueError(f"m must be in [1, {plan.max_m}] (the plan's max_m)")
    _shape(idx, (m, plan.top_k), "idx")
    _shape(wts, (m, plan.top_k), "wts")
    if not 0 <= int(layer) < plan.n_layers:
        raise ValueError("layer out of range")
    if y is None:
        y = torch.empty((m, plan.hidden), dtype=torch.float32, device=x.device)
    _shape(y, (m, plan.hidden), "y")
    check("moe_experts_routed", _lib.load().moe_experts_routed(
        plan.handle, int(layer), _dev_ptr(x2, "x"), _x_dtype(x2), m,
        _dev_ptr(idx, "idx", torch.int32), _dev_ptr(wts, "wts", torch.float32),
        _dev_ptr(y, "y", torch.float32), _stream()))
    return y


KERNEL_KINDS = ("route", "gate_up", "down", "combine", "layer")


class KernelTimes:
    """Per-kernel-kind accumulators of moe_expert_decode_profiled, indexed like
    KERNEL_KINDS: ms (sum of the dispatches' start-to-end times) and count."""

    def __init__(self):
        n = len(KERNEL_KINDS)
        self.ms = (ctypes.c_double * n)()
        self.count = (ctypes.c_int64 * n)()


def moe_expert_decode_profiled(plan: MoEPlan, x, y, acc: KernelTimes = None) -> KernelTimes:
    """One decode step with per-kernel start/stop events; accumulates into acc
    (a new KernelTimes when None) and returns it."""
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    _shape(x2, (x2.shape[0], plan.hidden), "x")
    _shape(y, (x2.shape[0], plan.hidden), "y")
    if not 1 <= x2.shape[0] <= plan.max_m:
        raise ValueError(f"m must be in [1, {plan.max_m}] (the plan's max_m)")
    if acc is None:
        acc = KernelTimes()
    check("moe_expert_decode_profiled", _lib.load().moe_expert_decode_profiled(
        plan.handle, _dev_ptr(x2, "x"), _x_dtype(x2), x2.shape[0], _dev_ptr(y, "y", torch.float32),
        acc.ms, acc.count, _stream()))
    return acc


LAYER_STAMPS = ("start", "routed", "gu_issued", "dn_issued", "gu_done", "h_stored", "barrier", "h_staged",
                "dn_done", "end")


def moe_expert_decode_timeline(plan: MoEPlan, x, y, n_blocks=4096):
    """One single-token step on the fused per-layer path with per-block phase
    stamps: returns a numpy uint64 array [L][blocks][16] of 100 MHz clock
    values (0 = phase not reached by that block), indexed by LAYER_STAMPS."""
    import numpy as np
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    _shape(x2, (1, plan.hidden), "x")
    _shape(y, (1, plan.hidden), "y")
    buf = np.zeros(plan.n_layers * n_blocks * 16, dtype=np.uint64)
    n = _lib.load().moe_expert_decode_timeline(
        plan.handle, _dev_ptr(x2, "x"), _x_dtype(x2), _dev_ptr(y, "y", torch.float32),
        buf.ctypes.data_as(ctypes.c_void_p), buf.size, _stream())
    if n < 0:
        check("moe_expert_decode_timeline", int(n))
    return buf[:n].reshape(plan.n_layers, -1, 16)


def stream_read(buf, n_blocks=0, sink=None):
    """Read every byte of buf with 16-byte loads; returns the per-block sink."""
    nb = n_blocks if n_blocks > 0 else 2048
    if sink is None:
        sink = torch.empty(nb, dtype=torch.float32, device=buf.device)
    elif sink.numel() < nb:
        raise ValueError("sink too small")
    check("bdg_stream_read", _lib.load().bdg_stream_read(
        _dev_ptr(buf, "buf"), buf.numel() * buf.element_size(), _dev_ptr(sink, "sink"), nb, _stream()))
    return sink


def stream_copy(src, dst):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    check("bdg_stream_copy", _lib.load().bdg_stream_copy(
        _dev_ptr(src, "src"), _dev_ptr(dst, "dst"), nbytes, _stream()))


def version():
    return _lib.load().bdg_version().decode()
