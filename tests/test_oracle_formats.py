"""Pins for the oracle's weight decoding, independent of the oracle's own code.

Each pin checks the oracle against something other than itself: the OCP MX
table, a bit-level construction of fp32 patterns, IEEE fp32 hardware
multiplies done by NumPy in float32, or hand-worked fixtures.  The mutation
tests at the end plant plausible mistakes in the oracle (on the CPU) and
check that a pin catches each one.
"""

import os

import numpy as np
import pytest

from oracle import formats, gemv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_e2m1_table():
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, v = line.split()
            vals.append((int(code), float(v)))
    assert [c for c, _ in vals] == list(range(16))
    return np.array([v for _, v in vals])


def e2m1_bits_construction(code):
    """fp32 bit pattern of an E2M1 code built field by field."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    if e == 0:
        mag = 0 if m == 0 else (126 << 23)          # 0 or 0.5
    else:
        mag = ((e - 1 + 127) << 23) | (m << 22)     # 2^(e-1) * (1 + m/2)
    return (s << 31) | mag


def f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ---------------------------------------------------------------- pins

def pin_e2m1(fm):
    got = fm.e2m1_value(np.arange(16))
    table = load_e2m1_table()
    assert np.array_equal(got, table)
    assert np.array_equal(np.signbit(got), np.signbit(table))      # code 8 is -0.0
    built = np.array([e2m1_bits_construction(c) for c in range(16)], dtype=np.uint32)
    assert np.array_equal(f32_bits(got), built)


def pin_e8m0(fm):
    e = np.arange(256)
    v = fm.e8m0_value(e)
    assert np.isnan(v[255]) and not np.any(np.isnan(v[:255]))
    assert v[127] == 1.0
    v32 = v[:255].astype(np.float32)
    bits = f32_bits(v32)
    assert bits[0] == 0x00400000                                   # 2^-127, fp32 subnormal
    assert np.array_equal(bits[1:], (np.arange(1, 255) << 23).astype(np.uint32))
    assert np.all(v[1:255] / v[:254] == 2.0)


def mxfp4_exhaustive_inputs():
    """256 rows (one per E8M0 byte), 32 columns = codes 0..15 twice."""
    codes_row = np.arange(16, dtype=np.uint8)
    packed = (codes_row[0::2] | (codes_row[1::2] << 4)).astype(np.uint8)   # 8 bytes = 16 codes
    codes = np.tile(np.concatenate([packed, packed]), (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None]
    return codes, scales


def pin_mxfp4_exhaustive(fm):
    codes, scales = mxfp4_exhaustive_inputs()
    got = fm.mxfp4_dequant(codes, scales)
    assert got.dtype == np.float32 and got.shape == (256, 32)
    # independent: IEEE fp32 multiply of the table value by the fp32 scale
    table32 = load_e2m1_table().astype(np.float32)
    scale32 = np.empty(256, dtype=np.float32)
    scale32[:255] = np.array([np.ldexp(np.float32(1), int(e) - 127) for e in range(255)],
                             dtype=np.float32)
    scale32[255] = np.float32(np.nan)
    with np.errstate(over="ignore", invalid="ignore"):
        want = np.tile(table32, 2)[None, :] * scale32[:, None]
    nan_got, nan_want = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_got, nan_want)
    assert np.array_equal(f32_bits(got)[~nan_got], f32_bits(want)[~nan_want])
    # spot checks of the special cases
    assert f32_bits(got[0, 1]) == 0x00200000        # 0.5 * 2^-127 = 2^-128, subnormal
    assert f32_bits(got[127, 8]) == 0x80000000      # -0.0 survives the scale
    assert np.isinf(got[254, 7]) and got[254, 7] > 0    # 6 * 2^127 overflows
    assert got[253, 5] == np.float32(3.0 * 2.0 ** 126)


def load_hand_mxfp4():
    blocks, fields = {}, {}
    with open(os.path.join(GOLDEN, "mxfp4_gemv_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            if p[0] == "block":
                blocks[(int(p[1]), int(p[2]))] = (int(p[3], 16), int(p[4]))
            else:
                fields.setdefault(p[0], []).append([float(t) for t in p[1:]])
    codes = np.zeros((2, 32), dtype=np.uint8)
    scales = np.zeros((2, 2), dtype=np.uint8)
    for (r, b), (byte, e) in blocks.items():
        codes[r, 16 * b:16 * (b + 1)] = byte
        scales[r, b] = e
    x = np.concatenate([np.ones(32), np.arange(32.0)])
    return codes, scales, x, fields


def pin_mxfp4_hand(fm, gm):
    codes, scales, x, fields = load_hand_mxfp4()
    w = fm.mxfp4_dequant(codes, scales)
    for r, c, v in fields["w"]:
        assert w[int(r), int(c)] == v
    y, den = gm.gemv(w, x)
    assert np.array_equal(y, np.array(fields["y"][0]))
    assert np.array_equal(den, np.array(fields["den"][0]))


def load_hand_int4():
    groups, fields = {}, {}
    with open(os.path.join(GOLDEN, "int4g_gemv_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            if p[0] == "group":
                groups[int(p[1])] = (int(p[2], 16), int(p[3], 16))
            elif p[0] == "zeros":
                fields["zeros"] = int(p[1], 16)
            else:
                fields.setdefault(p[0], []).append([float(t) for t in p[1:]])
    codes = np.zeros((1, 64), dtype=np.uint8)
    scales = np.zeros((1, 2), dtype=np.uint16)
    for g, (byte, s) in groups.items():
        codes[0, 32 * g:32 * (g + 1)] = byte
        scales[0, g] = s
    zeros = np.array([[fields["zeros"]]], dtype=np.uint8)
    return codes, scales, zeros, np.ones(128), fields


def pin_int4_hand(fm, gm):
    codes, scales, zeros, x, fields = load_hand_int4()
    w = fm.int4g_dequant(codes, scales, zeros, 64)
    for r, c, v in fields["w"]:
        assert w[int(r), int(c)] == v
    y, den = gm.gemv(w, x)
    assert y[0] == fields["y"][0][0] and den[0] == fields["den"][0][0]


def int4_exhaustive_inputs(scale_bits):
    """One row per fp16 scale; 16 groups of 32 (z = group index), q = 0..15 twice."""
    n = scale_bits.size
    q = np.arange(16, dtype=np.uint8)
    packed = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)
    codes = np.tile(np.tile(packed, 32), (n, 1))                 # 512 elements per row
    z = np.arange(16, dtype=np.uint8)
    zeros = np.tile((z[0::2] | (z[1::2] << 4)).astype(np.uint8), (n, 1))
    scales = np.repeat(scale_bits[:, None], 16, axis=1)
    return codes, scales, zeros


def pin_int4_exhaustive(fm, scale_bits):
    codes, scales, zeros = int4_exhaustive_inputs(scale_bits)
    got = fm.int4g_dequant(codes, scales, zeros, 32)
    # independent: fp32 hardware multiply of (q - z) by the fp16 scale widened to fp32
    q = np.tile(np.arange(16, dtype=np.float32), 32)
    z = np.repeat(np.arange(16, dtype=np.float32), 32)
    s32 = scale_bits.view(np.float16).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        want = (q - z)[None, :] * s32[:, None]
    nan_got, nan_want = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_got, nan_want)
    assert np.array_equal(f32_bits(got)[~nan_got], f32_bits(want)[~nan_want])


ALL_F16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


# ---------------------------------------------------------------- tests

def test_e2m1_table():
    pin_e2m1(formats)


def test_e8m0_closed_form():
    pin_e8m0(formats)


def test_mxfp4_dequant_exhaustive_4096():
    pin_mxfp4_exhaustive(formats)


def test_mxfp4_hand_worked_gemv():
    pin_mxfp4_hand(formats, gemv)


def test_int4_hand_worked_gemv():
    pin_int4_hand(formats, gemv)


@pytest.mark.parametrize("part", range(4))
def test_int4_dequant_exhaustive_all_fp16_scales(part):
    # 16 q x 16 z x all 65536 fp16 patterns (finite, inf, NaN), in 4 slices
    pin_int4_exhaustive(formats, ALL_F16[part * 16384:(part + 1) * 16384])


def test_int4_odd_group_count_zero_packing():
    # K = 96 with group 32 -> 3 groups, zeros row is 2 bytes, group 2 in a low nibble
    codes = np.full((1, 48), 0x77, dtype=np.uint8)            # q = 7 everywhere
    zeros = np.array([[0x21, 0x03]], dtype=np.uint8)           # z = 1, 2, 3
    scales = np.full((1, 3), 0x3C00, dtype=np.uint16)          # 1.0
    w = formats.int4g_dequant(codes, scales, zeros, 32)
    assert np.array_equal(w[0], np.repeat([6.0, 5.0, 4.0], 32).astype(np.float32))


def test_shape_validation():
    with pytest.raises(ValueError):
        formats.mxfp4_dequant(np.zeros((2, 8), np.uint8), np.zeros((2, 2), np.uint8))
    with pytest.raises(ValueError):
        formats.int4g_dequant(np.zeros((1, 48), np.uint8), np.zeros((1, 2), np.uint16),
                              np.zeros((1, 1), np.uint8), 64)


# ---------------------------------------------------------------- planted mistakes

_ORIG = {k: getattr(formats, k) for k in (
    "unpack_nibbles", "e2m1_value", "mxfp4_dequant", "int4g_dequant", "int4g_dequant64")}


class Mutant:
    """A copy of the formats namespace with one function replaced."""

    def __init__(self, **over):
        for name in dir(formats):
            if not name.startswith("__"):
                setattr(self, name, getattr(formats, name))
        for k, v in over.items():
            setattr(self, k, v)


def _swapped_nibbles(packed, count=None):
    out = _ORIG["unpack_nibbles"](packed, None)
    sw = out.copy()
    sw[..., 0::2], sw[..., 1::2] = out[..., 1::2], out[..., 0::2]
    return sw if count is None else sw[..., :count]


def _e2m1_bias0(code):
    code = np.asarray(code, dtype=np.int64)
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e))   # wrong bias
    return np.where(s == 1, -mag, mag)


def _e2m1_no_negzero(code):
    v = _ORIG["e2m1_value"](code)
    return np.where(v == 0, 0.0, v)


def _e8m0_bias128(e):
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(np.ones(e.shape), e - 128))


def _mxfp4_ftz(codes, scales):
    w = _ORIG["mxfp4_dequant"](codes, scales)
    tiny = np.abs(w) < np.float32(2.0 ** -126)
    return np.where(tiny, np.float32(0) * np.sign(w), w).astype(np.float32)


def _mxfp4_wrong_block_axis(codes, scales):
    # scale applied per 32 rows-worth instead of per 32 K-elements: block of the
    # transposed index
    n = codes.shape[0]
    vals = _ORIG["e2m1_value"](_ORIG["unpack_nibbles"](codes))
    s = formats.e8m0_value(scales)
    blk = np.repeat(s, 32, axis=1)[:, ::-1]          # blocks taken in the wrong order
    with np.errstate(over="ignore", invalid="ignore"):
        return (vals * blk[:n]).astype(np.float32)


def _int4_no_zero(codes, scales, zeros, group):
    return _ORIG["int4g_dequant"](codes, scales, np.zeros_like(zeros), group)


def _int4_zero_nibbles_swapped(codes, scales, zeros, group):
    z = ((zeros & 0x0F) << 4) | (zeros >> 4)
    return _ORIG["int4g_dequant"](codes, scales, z.astype(np.uint8), group)


def _int4_scale_in_f16(codes, scales, zeros, group):
    # product rounded in fp16 instead of exact
    w = _ORIG["int4g_dequant64"](codes, scales, zeros, group)
    with np.errstate(over="ignore", invalid="ignore"):
        return w.astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("pin,mut", [
    ("e2m1", dict(e2m1_value=_e2m1_bias0)),
    ("e2m1", dict(e2m1_value=_e2m1_no_negzero)),
    ("e8m0", dict(e8m0_value=_e8m0_bias128)),
    ("mx_exh", dict(mxfp4_dequant=_mxfp4_ftz)),
    ("mx_hand", dict(unpack_nibbles=_swapped_nibbles)),
    ("mx_hand", dict(mxfp4_dequant=_mxfp4_wrong_block_axis)),
    ("i4_hand", dict(int4g_dequant=_int4_no_zero)),
    ("i4_hand", dict(int4g_dequant=_int4_zero_nibbles_swapped)),
    ("i4_exh", dict(int4g_dequant=_int4_scale_in_f16)),
])
def test_planted_mistake_is_caught(pin, mut):
    # Functions inside formats call each other through the module, so mutants
    # that replace a helper are applied by patching the module temporarily.
    saved = {k: getattr(formats, k) for k in mut}
    try:
        for k, v in mut.items():
            setattr(formats, k, v)
        m = Mutant()
        with pytest.raises(AssertionError):
            if pin == "e2m1":
                pin_e2m1(m)
            elif pin == "e8m0":
                pin_e8m0(m)
            elif pin == "mx_exh":
                pin_mxfp4_exhaustive(m)
            elif pin == "mx_hand":
                pin_mxfp4_hand(m, gemv)
            elif pin == "i4_hand":
                pin_int4_hand(m, gemv)
            elif pin == "i4_exh":
                pin_int4_exhaustive(m, ALL_F16[15000:17000])
    finally:
        for k, v in saved.items():
            setattr(formats, k, v)
