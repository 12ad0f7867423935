"""Pins for the oracle's opt-in lossy activation modes (CPU only).

The quantizers are checked against an independent library routine (torch's
float8_e4m3fn conversion), a hand-worked rounding table from the E2M1 value
list (tests/golden/e2m1_rounding.txt), closed forms of the MX scale rule,
exact invariants (power-of-two shifts, idempotence, zero and non-finite
blocks), and the mode wiring of the layer (on-grid inputs are fixed points;
a mode never touches a projection format it does not name).
"""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import layer as OL
from oracle import lossy as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(v):
    """torch's own RNE conversion to float8_e4m3fn (inputs within +-448)."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- rounding
def test_e4m3_rounding_matches_torch_on_grid_midpoints_and_random():
    mags = F.e4m3_value(np.arange(0x7F))
    mids = (mags[:-1] + mags[1:]) / 2
    rng = np.random.default_rng(7)
    rnd = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-14, 1, 20000))
    v = np.concatenate([mags, -mags, mids, -mids, mids * (1 + 2 ** -20), mids * (1 - 2 ** -20), rnd])
    v = v.astype(np.float32).astype(np.float64)     # values torch sees exactly
    assert np.array_equal(Q.round_to_element(v, "e4m3"), _torch_e4m3(v))


def test_e4m3_rounding_saturates():
    assert Q.round_to_element(np.array([464.0, 479.9, 1e6]), "e4m3").tolist() == [0x7E] * 3
    assert Q.round_to_element(np.array([-1e6]), "e4m3").tolist() == [0xFE]


def test_e2m1_rounding_table():
    vals, want = [], []
    with open(os.path.join(GOLDEN, "e2m1_rounding.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, c = line.split()
                vals.append(float(a))
                want.append(int(c, 16))
    assert Q.round_to_element(np.array(vals), "e2m1").tolist() == want


def test_grid_values_round_trip():
    for elem, dec, n in (("e4m3", F.e4m3_value, 0x7F), ("e2m1", F.e2m1_value, 8)):
        codes = np.arange(n)
        assert np.array_equal(Q.round_to_element(dec(codes), elem), codes)
        neg = codes | (0x80 if elem == "e4m3" else 0x8)
        assert np.array_equal(Q.round_to_element(dec(neg), elem), neg)


# ---------------------------------------------------------------- MX scale rule
def test_mx_unit_block_closed_form():
    v = np.ones((1, 32))
    c8, s8 = Q.mx_quantize(v, "e4m3")   # shared = 0 - 8: 1.0 -> 256 = 2^8, E4M3 0x78
    assert s8.tolist() == [[119]] and np.all(c8 == 0x78)
    c4, s4 = Q.mx_quantize(v, "e2m1")   # shared = 0 - 2: 1.0 -> 4.0, E2M1 0x6
    assert s4.tolist() == [[125]] and np.all(c4 == 0x6)


def test_mx_saturating_block():
    v = np.zeros((1, 32))
    v[0, 3] = 1.9                      # floor(log2 1.9) = 0
    c8, s8 = Q.mx_quantize(v, "e4m3")  # 1.9 * 2^8 = 486.4 -> 448
    assert s8[0, 0] == 119 and c8[0, 3] == 0x7E and np.all(np.delete(c8[0], 3) == 0)
    c4, s4 = Q.mx_quantize(-v, "e2m1")  # -1.9 * 4 = -7.6 -> -6
    assert s4[0, 0] == 125 and c4[0, 3] == 0xF


def test_mx_scale_range_clamps():
    big = np.full((1, 32), 3.3895313892515355e38)   # largest bf16: floor(log2) = 127
    _, s = Q.mx_quantize(big, "e4m3")
    assert s[0, 0] == 127 + 127 - 8
    tiny = np.full((1, 32), 2.0 ** -133)              # smallest bf16 subnormal
    c, s = Q.mx_quantize(tiny, "e4m3")
    assert s[0, 0] == 0 and np.all(c == 0x08)         # 2^-133 / 2^-127 = 2^-6


def test_mx_zero_and_nonfinite_blocks():
    v = np.zeros((2, 64))
    v[1, 40] = np.nan
    v[1, 5] = 1.5
    for elem in ("e4m3", "e2m1"):
        c, s = Q.mx_quantize(v, elem)
        assert s[0].tolist() == [0, 0] and np.all(c[0] == 0)
        assert s[1, 1] == 255 and np.all(c[1, 32:] == 0)
        assert s[1, 0] != 255 and c[1, 5] != 0
    v[1, 40] = -np.inf
    assert Q.mx_quantize(v, "e4m3")[1][1, 1] == 255


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
def test_mx_power_of_two_shift_and_idempotence(elem):
    rng = np.random.default_rng(3)
    v = OL.bf16_value(synth.bf16_bits_from_f32(rng.standard_normal((16, 256)).astype(np.float32)))
    c, s = Q.mx_quantize(v, elem)
    for j in (-20, -1, 3, 17):
        c2, s2 = Q.mx_quantize(v * 2.0 ** j, elem)
        assert np.array_equal(c2, c) and np.array_equal(s2.astype(int), s.astype(int) + j)
    d = Q.mx_dequantize(c, s, elem)
    c3, s3 = Q.mx_quantize(d, elem)
    assert np.array_equal(Q.mx_dequantize(c3, s3, elem), d)


@pytest.mark.parametrize("elem,rel", [("e4m3", 2.0 ** -4), ("e2m1", 2.0 ** -2)])
def test_mx_error_bound(elem, rel):
    """Rounding error of a normal element is at most half a quantum (rel of
    |v|); below the normal range it is half the subnormal quantum; a
    saturated element errs by its excess over the largest element value."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-6, 6, (64, 1)))
    c, s = Q.mx_quantize(v, elem)
    d = Q.mx_dequantize(c, s, elem)
    X = np.repeat(F.e8m0_value(s), 32, axis=1)
    emax_val, sub_q = (448.0, 2.0 ** -9) if elem == "e4m3" else (6.0, 0.5)
    bound = np.maximum(rel * np.abs(v), 0.5 * sub_q * X) + np.maximum(np.abs(v) - emax_val * X, 0)
    assert np.all(np.abs(v - d) <= bound * (1 + 1e-12))


# ---------------------------------------------------------------- per-token 1x128
def test_t128_unit_scale_matches_torch():
    rng = np.random.default_rng(11)
    v = rng.uniform(-448, 448, (4, 256))
    v[:, 0] = 448.0
    v[:, 128] = -448.0
    v = OL.bf16_value(synth.bf16_bits_from_f32(v.astype(np.float32)))
    c, s = Q.t128_quantize(v)
    assert np.all(s == 1.0)                       # 448 / 448
    assert np.array_equal(c, _torch_e4m3(v))


def test_t128_scale_and_ragged_tail():
    rng = np.random.default_rng(12)
    v = OL.bf16_value(synth.bf16_bits_from_f32(rng.standard_normal((3, 300)).astype(np.float32)))
    c, s = Q.t128_quantize(v)
    assert c.shape == (3, 300) and s.shape == (3, 3)
    for b, (lo, hi) in enumerate([(0, 128), (128, 256), (256, 300)]):
        amax = np.max(np.abs(v[:, lo:hi]), axis=1).astype(np.float32)
        assert np.array_equal(s[:, b], amax / np.float32(448))
        i = np.argmax(np.abs(v[:, lo:hi]), axis=1)
        top = c[np.arange(3), lo + i] & 0x7F
        assert np.all(top == 0x7E)                # the block maximum maps to 448
    d = Q.t128_dequantize(c, s)
    assert np.all(np.abs(d - v) <= 2.0 ** -4 * np.abs(v) + 2.0 ** -10 * np.repeat(s, 128, 1)[:, :300])


def test_t128_zero_and_nonfinite():
    v = np.zeros((2, 128))
    v[1, 7] = np.inf
    c, s = Q.t128_quantize(v)
    assert np.all(c == 0)
    assert s[0, 0] == np.float32(2.0 ** -64) / np.float32(448) and np.isnan(s[1, 0])


# ---------------------------------------------------------------- layer wiring
def _small_layer(fmt, shared_fmt=None, seed=0):
    w = synth.Workload("t", T=6, H=256, E=6, I=128, top_k=2, fmt=fmt,
                       I_shared=128 if shared_fmt else 0, shared_fmt=shared_fmt, seed=seed)
    return w, synth.make_layer(w, workers=1)


def test_mode_leaves_other_formats_exact():
    w, L = _small_layer(synth.FMT_NVFP4, synth.FMT_FP8)
    x = synth.make_x(w)
    ref = OL.layer_forward(L, x)
    for mode in ("mxfp8", "mxfp4"):
        got = Q.layer_forward(L, x, mode)
        assert np.array_equal(got.out64, ref.out64)
    got = Q.layer_forward(L, x, "fp8_t128")       # quantizes the FP8 shared expert only
    assert np.array_equal(got.y, ref.y) and not np.array_equal(got.out64, ref.out64)


@pytest.mark.parametrize("mode,elem", [("mxfp8", "e4m3"), ("mxfp4", "e2m1")])
def test_on_grid_activations_are_fixed_points(mode, elem):
    """x already on the mode's grid: gate/up sees x unchanged, so h equals the
    exact chain's h; the down input h is then quantized."""
    w, L = _small_layer(synth.FMT_MXFP4)
    x = synth.make_x(w)
    xv = OL.bf16_value(x)
    xg = Q.mx_dequantize(*Q.mx_quantize(xv, elem), elem)
    xb = OL.bf16_bits(xg)
    assert np.array_equal(OL.bf16_value(xb), xg)   # the grid is bf16-exact
    ref = OL.layer_forward(L, xb)
    got = Q.layer_forward(L, xb, mode)
    assert np.array_equal(got.h, ref.h)
    assert not np.array_equal(got.y, ref.y)
    dec = OL._Decoded(L)
    for t in range(2):
        for j in range(w.top_k):
            e = int(ref.routing.ids[t, j])
            hq = Q.quantize_input(ref.h[t, j][None], mode)[0]
            assert np.allclose(got.y[t, j], dec("down", e) @ hq, rtol=1e-12, atol=1e-14)
