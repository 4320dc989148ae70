"""The C ABI without a GPU: libbdg.so loads, exports every function that
include/bdg.h declares, the binding covers each of them, and the pure host
entry points (status text, version, workspace sizes, argument rejection before
any launch) behave as the header states.  No call here reaches a kernel."""

import ctypes
import os
import re

import pytest

from bit_dequant_gemv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bdg.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^(?:const\s+char\s*\*|int64_t|int)\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_parses():
    names = _declared()
    assert "attn_decode" in names and "qgemv" in names and len(names) >= 20


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), f"libbdg.so does not export {name}"


def test_binding_covers_the_header():
    assert sorted(_lib.EXPORTED) == _declared()
    lib = _lib.load()
    for name in _lib.EXPORTED:
        assert getattr(lib, name).argtypes is not None or name == "bdg_version"


def test_status_text_and_version():
    lib = _lib.load()
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.bdg_strerror(st)
    assert lib.bdg_version().decode()


def test_attention_workspace_sizes():
    lib = _lib.load()
    part = 64 * 8 * 8 * 66 * 4            # up to 64 splits x 8 kv heads x 8 heads x (max, sum, 64 values)
    assert lib.attn_decode_workspace(64, 8, 64, 1, 128) == part
    assert lib.attn_decode_workspace(64, 8, 64, 1, 1 << 20) == part
    assert lib.attn_decode_workspace(64, 8, 64, 3, 8192) == 3 * part
    assert lib.attn_decode_workspace(16, 2, 64, 1, 8192) == part // 4
    # shapes the kernel does not take
    assert lib.attn_decode_workspace(64, 8, 128, 1, 8192) == -1
    assert lib.attn_decode_workspace(32, 8, 64, 1, 8192) == -1
    assert lib.attn_decode_workspace(64, 8, 64, 0, 8192) == -1


def test_attention_rejects_arguments_before_launch():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)        # never dereferenced: every call below fails its checks
    args = dict(q=fake, k=fake, v=fake, kc=fake, vc=fake, dt=1, cap=256, hq=64, hkv=8, d=64, m=1, pos0=10,
                tab=fake, rows=256, sm=0.125, sinks=None, window=0, o=fake, ws=fake, wsb=1 << 30, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return lib.attn_decode(a["q"], a["k"], a["v"], a["kc"], a["vc"], a["dt"], a["cap"], a["hq"], a["hkv"],
                               a["d"], a["m"], a["pos0"], a["tab"], a["rows"], a["sm"], a["sinks"], a["window"],
                               a["o"], a["ws"], a["wsb"], a["s"])
    assert call(q=None) == _lib.BDG_E_INVALID
    assert call(dt=7) == _lib.BDG_E_INVALID
    assert call(pos0=256) == _lib.BDG_E_INVALID           # past the cache
    assert call(rows=5) == _lib.BDG_E_INVALID             # past the rotary table
    assert call(sm=0.0) == _lib.BDG_E_INVALID
    assert call(window=-1) == _lib.BDG_E_INVALID
    assert call(d=128) == _lib.BDG_E_UNSUPPORTED
    assert call(hq=16) == _lib.BDG_E_UNSUPPORTED
    assert call(m=65, cap=1000, rows=1000) == _lib.BDG_E_UNSUPPORTED
    assert call(q=ctypes.c_void_p(0x1004)) == _lib.BDG_E_ALIGN
    assert call(ws=None) == _lib.BDG_E_INVALID             # the workspace is required
    assert call(ws=fake, wsb=100) == _lib.BDG_E_INVALID    # and must be large enough


def test_rope_table_rejects_arguments_before_launch():
    lib = _lib.load()
    good = dict(theta=150000.0, factor=32.0, beta_fast=32.0, beta_slow=1.0, orig_ctx=4096, truncate=0)
    fake = ctypes.c_void_p(0x1000)
    for bad in (dict(theta=1.0), dict(factor=0.0), dict(orig_ctx=0), dict(truncate=2)):
        r = _lib.Rope(**dict(good, **bad))
        assert lib.attn_rope_table(ctypes.byref(r), 64, 16, fake, None, None, None) == _lib.BDG_E_INVALID
    r = _lib.Rope(**good)
    assert lib.attn_rope_table(ctypes.byref(r), 63, 16, fake, None, None, None) == _lib.BDG_E_INVALID
    assert lib.attn_rope_table(ctypes.byref(r), 64, 0, fake, None, None, None) == _lib.BDG_E_INVALID


def test_prefill_workspace_size_is_host_arithmetic():
    lib = _lib.load()
    assert lib.moe_prefill_mx_workspace(64, 2880, 2880, 32, 4) > 0
    assert lib.moe_prefill_mx_workspace(0, 2880, 2880, 32, 4) == -1


def test_mx_gemm_workspace_size():
    """Two 256-byte aligned parts of stage-major scale words: [k/128][n] and
    [k/128][m] (k/128 rounded up: K = 2880 is 90 blocks, 23 stages)."""
    lib = _lib.load()
    a256 = lambda b: (b + 255) // 256 * 256
    assert lib.mx_gemm_workspace(5760, 2880, 4096) == a256(4 * 23 * 5760) + a256(4 * 23 * 4096)
    assert lib.mx_gemm_workspace(1, 32, 1) == 2 * 256
    assert lib.mx_gemm_workspace(5760, 2880, 0) == -1
    assert lib.mx_gemm_workspace(5760, 48, 8) == -1


def _fake_mx(n=256, k=256, **kw):
    return _lib.QMat(fmt=_lib.BDG_FMT_MXFP4, group=32, n=n, k=k, codes=0x100000000, scales=0x200000000,
                     zeros=None, expert_stride_codes=kw.get("sc", 0), expert_stride_scales=kw.get("ss", 0),
                     expert_stride_zeros=0)


def test_mx_scale_words_size_and_rejections():
    """Stage-major scale words: E * ceil(k/128) * n 32-bit words; the staging
    call rejects bad arguments before any launch (fake device addresses)."""
    lib = _lib.load()
    qm = _fake_mx(5760, 2880)
    assert lib.mx_scale_words_bytes(ctypes.byref(qm), 32) == 4 * 32 * 23 * 5760
    assert lib.mx_scale_words_bytes(ctypes.byref(_fake_mx(3, 32)), 1) == 4 * 3
    assert lib.mx_scale_words_bytes(ctypes.byref(qm), 0) == -1
    i4 = _lib.QMat(fmt=_lib.BDG_FMT_INT4G, group=64, n=256, k=256, codes=0x100000000, scales=0x200000000,
                   zeros=0x300000000)
    assert lib.mx_scale_words_bytes(ctypes.byref(i4), 1) == -1
    need = lib.mx_scale_words_bytes(ctypes.byref(_fake_mx()), 1)
    out = 0x700000000
    assert lib.mx_stage_scales(ctypes.byref(i4), 1, out, 1 << 20, None) == _lib.BDG_E_INVALID
    assert lib.mx_stage_scales(ctypes.byref(_fake_mx()), 1, None, need, None) == _lib.BDG_E_INVALID
    assert lib.mx_stage_scales(ctypes.byref(_fake_mx()), 1, out, need - 1, None) == _lib.BDG_E_INVALID
    assert lib.mx_stage_scales(ctypes.byref(_fake_mx()), 1, out + 4, need, None) == _lib.BDG_E_ALIGN
    # several experts need their strides
    assert lib.mx_stage_scales(ctypes.byref(_fake_mx()), 2, out, 2 * need, None) == _lib.BDG_E_INVALID


def test_mx_gemm_rejects_misaligned_scale_words():
    lib = _lib.load()
    qm = _fake_mx()
    qm.mx_scale_words = 0x800000004
    need = lib.mx_gemm_workspace(256, 256, 64)
    assert lib.mx_gemm(ctypes.byref(qm), 0x300000000, 0x400000000, 64, 0x500000000, 0x600000000, need,
                       None) == _lib.BDG_E_ALIGN


def test_mx_gemm_rejects_a_short_workspace():
    """Fake device addresses, never dereferenced: the size check fails first."""
    lib = _lib.load()
    qm = _lib.QMat(fmt=_lib.BDG_FMT_MXFP4, group=32, n=256, k=256, codes=0x100000000, scales=0x200000000,
                   zeros=None, expert_stride_codes=0, expert_stride_scales=0, expert_stride_zeros=0)
    need = lib.mx_gemm_workspace(256, 256, 64)
    args = (ctypes.byref(qm), 0x300000000, 0x400000000, 64, 0x500000000, 0x600000000)
    assert lib.mx_gemm(*args, need - 1, None) == _lib.BDG_E_INVALID
    assert lib.mx_gemm(ctypes.byref(qm), 0x300000000, 0x400000000, 64, 0x500000000, None, need, None) == \
        _lib.BDG_E_INVALID
    assert lib.mx_gemm(ctypes.byref(qm), 0x300000000, 0x400000000, 64, 0x500000000, 0x600000008, need, None) == \
        _lib.BDG_E_ALIGN


@pytest.mark.parametrize("name", ["mxfp4_dequant", "qgemv", "moe_router_topk", "mx_gemm"])
def test_null_arguments_are_rejected(name):
    lib = _lib.load()
    fn = getattr(lib, name)
    nargs = len(fn.argtypes)
    zero = [None if t is ctypes.c_void_p or issubclass(t, ctypes._Pointer) else 0 for t in fn.argtypes]
    assert fn(*zero[:nargs]) == _lib.BDG_E_INVALID


def _plan_desc(k=4, E=32, H=2880, I=2880, L=1, max_m=1, flags=0, mutate=None):
    """A plan descriptor over fake device addresses (never dereferenced: every
    case below fails its host checks before any HIP call)."""
    layers = (_lib.LayerDesc * L)()
    for l in range(L):
        base = 0x100000000 * (l + 1)

        def qmat(n, kk, off):
            return _lib.QMat(fmt=_lib.BDG_FMT_MXFP4, group=32, n=n, k=kk, codes=base + off,
                             scales=base + off + 0x40000000, zeros=None,
                             expert_stride_codes=n * kk // 2, expert_stride_scales=n * kk // 32,
                             expert_stride_zeros=0)
        layers[l].w_router = base
        layers[l].b_router = None
        layers[l].gate_up = qmat(2 * I, H, 0x1000000)
        layers[l].down = qmat(H, I, 0x8000000)
    if mutate:
        mutate(layers)
    return _lib.MoEDesc(n_layers=L, hidden=H, inter=I, n_experts=E, top_k=k, fmt=_lib.BDG_FMT_MXFP4,
                        group=32, flags=flags, norm_eps=1e-5, max_m=max_m, layers=layers), layers


def _create(desc):
    lib = _lib.load()
    handle = ctypes.c_void_p()
    st = lib.moe_plan_create(ctypes.byref(desc), ctypes.byref(handle))
    assert handle.value is None, "a rejected plan must not be returned"
    return st


def test_plan_create_rejects_arguments_before_any_allocation():
    lib = _lib.load()
    assert lib.moe_plan_create(None, None) == _lib.BDG_E_INVALID
    d, _ = _plan_desc(k=33, E=32)
    assert _create(d) == _lib.BDG_E_INVALID                 # k > E
    d, _ = _plan_desc(k=0)
    assert _create(d) == _lib.BDG_E_INVALID                 # k < 1
    d, _ = _plan_desc(max_m=0)
    assert _create(d) == _lib.BDG_E_INVALID
    d, _ = _plan_desc(max_m=17)
    assert _create(d) == _lib.BDG_E_UNSUPPORTED             # past BDG_MAX_M
    d, _ = _plan_desc(H=2890)
    assert _create(d) == _lib.BDG_E_INVALID                 # H % 32
    d, _ = _plan_desc(flags=128)
    assert _create(d) == _lib.BDG_E_INVALID                 # unknown flag

    def zero_stride_codes(ls):
        ls[0].gate_up.expert_stride_codes = 0
    d, _ = _plan_desc(mutate=zero_stride_codes)
    assert _create(d) == _lib.BDG_E_INVALID                 # experts would alias

    def zero_stride_scales(ls):
        ls[0].down.expert_stride_scales = 0
    d, _ = _plan_desc(mutate=zero_stride_scales)
    assert _create(d) == _lib.BDG_E_INVALID

    def misaligned_codes(ls):
        ls[0].down.codes += 8
    d, _ = _plan_desc(mutate=misaligned_codes)
    assert _create(d) == _lib.BDG_E_ALIGN

    def misaligned_stride(ls):
        ls[0].gate_up.expert_stride_codes += 4
    d, _ = _plan_desc(mutate=misaligned_stride)
    assert _create(d) == _lib.BDG_E_ALIGN

    def wrong_shape(ls):
        ls[0].down.n = 2848
    d, _ = _plan_desc(mutate=wrong_shape)
    assert _create(d) == _lib.BDG_E_INVALID

    def no_router(ls):
        ls[0].w_router = None
    d, _ = _plan_desc(mutate=no_router)
    assert _create(d) == _lib.BDG_E_INVALID


def test_decode_calls_reject_a_null_plan():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_expert_decode(None, fake, 0, 1, fake, None, None, None, None) == _lib.BDG_E_INVALID
    assert lib.moe_experts_routed(None, 0, fake, 0, 1, fake, fake, fake, None) == _lib.BDG_E_INVALID
    assert lib.moe_plan_destroy(None) == _lib.BDG_OK


def test_qgemv_rejects_matrices_past_32_bit_offsets():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    # 2^21 rows x 4096 columns: 2^32 code bytes, one past what 32-bit offsets reach
    big = _lib.QMat(fmt=_lib.BDG_FMT_MXFP4, group=32, n=1 << 21, k=4096, codes=0x100000000,
                    scales=0x200000000, zeros=None, expert_stride_codes=0, expert_stride_scales=0,
                    expert_stride_zeros=0)
    assert lib.qgemv(ctypes.byref(big), fake, 0, 1, fake, None) == _lib.BDG_E_UNSUPPORTED
