"""Pins for the oracle's format decoders (CPU only).

Each decoder is checked against something other than itself: the format
specifications' value tables (tests/golden/), torch's own float8 conversions
(an independent library routine), hand-worked examples, and a round trip
through the generator's separately written encoders.
"""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            out[int(c, 16)] = float(v)
    return out


def _same(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return np.all((a == b) & (np.signbit(a) == np.signbit(b)) | (np.isnan(a) & np.isnan(b)))


def test_e2m1_all_codes_match_spec_table():
    table = _read_golden("e2m1_values.txt")
    assert sorted(table) == list(range(16))
    got = F.e2m1_value(np.arange(16))
    assert _same(got, [table[c] for c in range(16)])


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = F.e4m3_value(np.arange(256))
    assert _same(got, ref)


def test_e4m3_spec_anchors():
    for c, v in _read_golden("fp8_e4m3_anchors.txt").items():
        assert _same(F.e4m3_value(c), v), hex(c)


def test_e8m0_all_codes_match_torch_and_spec():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float32).double().numpy()
    got = F.e8m0_value(np.arange(256))
    assert _same(got, ref)
    for c, v in _read_golden("e8m0_anchors.txt").items():
        assert _same(F.e8m0_value(c), v), hex(c)


def test_nibble_order_low_nibble_is_even_index():
    # byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    assert list(F.unpack_nibbles(np.array([[0x21, 0xF7]], np.uint8))[0]) == [1, 2, 7, 15]


def test_nvfp4_hand_worked_block():
    # one row, 32 columns = two 16-blocks.  Block 0: every code 0x3 (1.5) with
    # scale 0x40 (e=8,m=0 -> 2.0); block 1: codes alternate 0x7 (6) / 0xF (-6),
    # scale 0x01 (2^-9).  Tensor scale 0.25.
    codes = np.zeros((1, 16), np.uint8)
    codes[0, :8] = 0x33
    codes[0, 8:] = 0xF7
    scales = np.array([[0x40, 0x01]], np.uint8)
    w = F.dequant_nvfp4(codes, scales, 0.25)
    assert np.all(w[0, :16] == 1.5 * 2.0 * 0.25)
    assert np.all(w[0, 16::2] == 6 * 2.0 ** -9 * 0.25)
    assert np.all(w[0, 17::2] == -6 * 2.0 ** -9 * 0.25)


def test_mxfp4_hand_worked_block():
    codes = np.zeros((2, 32), np.uint8)
    codes[0, :] = 0x52          # element0 code 2 (1.0), element1 code 5 (3.0)
    codes[1, :] = 0x9C          # element0 code 0xC (-2.0), element1 code 9 (-0.5)
    scales = np.array([[127 + 3, 127 - 2], [0, 0xFF]], np.uint8)
    w = F.dequant_mxfp4(codes, scales)
    assert np.all(w[0, 0:32:2] == 8.0) and np.all(w[0, 1:32:2] == 24.0)
    assert np.all(w[0, 32::2] == 0.25) and np.all(w[0, 33::2] == 0.75)
    assert np.all(w[1, 0:32:2] == -2.0 * 2.0 ** -127)
    assert np.all(np.isnan(w[1, 32:]))


def test_mxfp8_hand_worked_block():
    codes = np.zeros((2, 64), np.uint8)
    codes[0, :32] = 0x38        # 1.0
    codes[0, 32:] = 0xC0        # -2.0
    codes[1, :32] = 0x7E        # 448
    codes[1, 40] = 0x7F         # NaN code
    codes[1, 33] = 0x01         # smallest subnormal, 2^-9
    scales = np.array([[127 + 3, 127 - 2], [127, 127 + 1]], np.uint8)
    w = F.dequant_mxfp8(codes, scales)
    assert np.all(w[0, :32] == 8.0) and np.all(w[0, 32:] == -0.5)
    assert np.all(w[1, :32] == 448.0) and np.isnan(w[1, 40])
    assert w[1, 33] == 2.0 ** -8 and w[1, 34] == 0.0
    scales[0, 0] = 0xFF
    assert np.all(np.isnan(F.dequant_mxfp8(codes, scales)[0, :32]))


def test_fp8_b128_edge_blocks():
    rows, cols = 130, 200
    codes = np.full((rows, cols), 0x38, np.uint8)      # 1.0 everywhere
    codes[129, 199] = 0xC0                             # -2.0
    scales = np.array([[1.0, 2.0], [3.0, 0.5]], np.float32)
    w = F.dequant_fp8_b128(codes, scales)
    assert w[0, 0] == 1.0 and w[127, 127] == 1.0
    assert w[0, 128] == 2.0 and w[127, 199] == 2.0
    assert w[128, 0] == 3.0 and w[129, 127] == 3.0
    assert w[128, 128] == 0.5 and w[129, 199] == -1.0


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_round_trip_through_generator_encoders(fmt):
    """Decode(encode(w)) lies within half a code step of w everywhere."""
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[3, :16] = 0.0                                   # an all-zero block
    qw = synth.QWeight(fmt, 256, 384, 1, *_encode(fmt, w))
    d = F.dequant(qw, 0)
    if fmt == synth.FMT_FP8:
        # E4M3 keeps 4 significant bits: rel. error <= 2^-4 (plus subnormal quantum)
        s = np.repeat(np.repeat(qw.scales[0], 128, 0), 128, 1)[:256, :384]
        assert np.all(np.abs(d - w) <= np.abs(w) * 2.0 ** -4 + s * 2.0 ** -10)
    elif fmt == synth.FMT_MXFP8:
        # E4M3 rounding plus saturation: the OCP shared exponent leaves
        # |w|/s in [256, 512) for the block maximum, clamped to 448
        s = np.repeat(F.e8m0_value(qw.scales[0]), 32, axis=1)
        sat = np.maximum(0.0, np.abs(w) - 448.0 * s)
        assert np.all(np.abs(d - w) <= np.abs(w) * 2.0 ** -4 + s * 2.0 ** -10 + sat + 1e-15)
        assert np.all(sat <= np.abs(w) / 8)
    else:
        blk = 16 if fmt == synth.FMT_NVFP4 else 32
        if fmt == synth.FMT_NVFP4:
            s = F.e4m3_value(qw.scales[0]) * float(qw.tensor_scale[0])
        else:
            s = F.e8m0_value(qw.scales[0])
        s = np.repeat(s, blk, axis=1)
        # Half the widest E2M1 gap (4 -> 6) is one scale unit.  Codes saturate
        # at 6: for MXFP4 by construction (the OCP shared exponent leaves
        # |w|/s in [4, 8) for the block maximum), for NVFP4 only when the E4M3
        # block scale itself rounded down (by at most 2^-4 relative).
        sat = np.maximum(0.0, np.abs(w) - 6.0 * s)
        assert np.all(np.abs(d - w) <= s + sat + 1e-12)
        if fmt == synth.FMT_NVFP4:
            assert np.all(sat <= np.abs(w) * 2.0 ** -4)
    assert np.all(d[3, :16] == 0.0)
    # the decode must also be close in aggregate (catches sign/order mistakes)
    assert np.linalg.norm(d - w) / np.linalg.norm(w) < 0.15


def _encode(fmt, w):
    if fmt == synth.FMT_NVFP4:
        c, s, ts = synth.encode_nvfp4(w)
        return c[None], s[None], np.array([ts], np.float32)
    if fmt == synth.FMT_MXFP4:
        c, s = synth.encode_mxfp4(w)
        return c[None], s[None], None
    if fmt == synth.FMT_MXFP8:
        c, s = synth.encode_mxfp8(w)
        return c[None], s[None], None
    c, s = synth.encode_fp8_b128(w)
    return c[None], s[None], None
