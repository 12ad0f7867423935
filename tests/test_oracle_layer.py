"""Pins for the oracle's layer steps (CPU only).

Each step is checked against an independent route to the same answer: exact
rational arithmetic (fractions), correctly rounded sums (math.fsum), pure
Python brute force, closed forms, torch's own bf16 rounding, and special
cases that reduce to a plain dense MLP.  A dropped term, wrong sign, wrong
index or transposed operand in the oracle fails at least one of these.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import layer as O

TINY = synth.WORKLOADS["tiny_nvfp4_t4"]


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------
def _all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        v = (bits << 16).view(np.float32).astype(np.float64)
    fin = np.isfinite(v) & ~np.signbit(v)
    vals = np.unique(v[fin])
    return vals, bits[fin][np.unique(v[fin], return_index=True)[1]]


def test_bf16_value_matches_torch_on_every_pattern():
    """bf16_value against torch's own bfloat16 -> float64 conversion, all
    65,536 bit patterns (NaN patterns compared as NaN, signed zeros by sign)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_value(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # anchors: 1.0, -2.0, the largest finite, the smallest subnormal, +inf
    assert O.bf16_value(np.uint16(0x3F80)) == 1.0
    assert O.bf16_value(np.uint16(0xC000)) == -2.0
    assert O.bf16_value(np.uint16(0x7F7F)) == (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert O.bf16_value(np.uint16(0x0001)) == 2.0 ** -133
    assert O.bf16_value(np.uint16(0x7F80)) == math.inf


def test_round_bf16_brute_force_nearest_ties_even():
    vals, bits = _all_bf16_values()           # every non-negative finite bf16
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(4000) * np.exp2(rng.integers(-140, 128, 4000)),
        (vals[1:200] + vals[:199]) / 2,        # exact midpoints (ties)
        [vals[-1] * (1 + 2.0 ** -9), vals[-1] * (1 + 2.0 ** -8.5), 0.0, 2.0 ** -134, 3 * 2.0 ** -134],
    ])
    got = O.round_bf16(x)
    for xi, gi in zip(x, got):
        a = abs(xi)
        if a >= vals[-1] + 2.0 ** 119:         # overflow midpoint: max + half ulp
            assert gi == math.copysign(math.inf, xi)
            continue
        i = np.searchsorted(vals, a)
        cands = [vals[j] for j in (i - 1, i) if 0 <= j < len(vals)]
        d = [abs(a - c) for c in cands]
        best = [c for c, dd in zip(cands, d) if dd == min(d)]
        if len(best) > 1:   # tie: even mantissa (low bit of the bf16 pattern clear)
            best = [c for c in best if (int(bits[np.searchsorted(vals, c)]) & 1) == 0]
        assert gi == math.copysign(best[0], xi), (xi, gi, best)


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-130, 120, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# SwiGLU activation
# ---------------------------------------------------------------------------
def test_silu_closed_forms():
    g = np.linspace(-30, 30, 1001)
    s = O.silu(g)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(s - O.silu(-g), g, rtol=0, atol=1e-12)      # silu(g) - silu(-g) = g
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15
    assert O.silu(np.array([-1000.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------
def test_router_logits_vs_exact_rationals():
    L = synth.make_layer(TINY)
    x = synth.make_x(TINY)
    l, bound = O.router_logits(x, L.router_w, L.router_bias)
    xv = O.bf16_value(x)
    for t in range(x.shape[0]):
        for e in range(L.E):
            exact = sum(Fraction(float(xv[t, h])) * Fraction(float(L.router_w[h, e])) for h in range(L.H))
            assert abs(Fraction(l[t, e]) - exact) <= Fraction(bound[t])
            assert abs(l[t, e] - float(exact)) <= 1e-12 * (1 + abs(float(exact)))
        row = O.exact_logits_row(x[t], L.router_w, L.router_bias)
        for e in range(L.E):
            exact = sum(Fraction(float(xv[t, h])) * Fraction(float(L.router_w[h, e])) for h in range(L.H))
            assert row[e] == float(exact)          # correctly rounded


def _brute_topk(l_row, k):
    keyed = sorted(range(len(l_row)),
                   key=lambda e: (1 if math.isnan(l_row[e]) else 0,
                                  0.0 if math.isnan(l_row[e]) else -l_row[e], e))
    return keyed[:k]


def test_topk_brute_force_with_ties_and_nans():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((50, 16)).astype(np.float32)
    logits[0, [3, 7, 11]] = 9.5                 # exact ties -> lower id first
    logits[1, :] = 1.0                          # all tied
    logits[2, [0, 5]] = np.nan                  # NaN after every number
    logits[3, :] = np.nan
    logits[3, 9] = -np.inf
    logits[4, 2] = np.inf
    ids, w = O.route_from_logits(logits, 5, True)
    for t in range(logits.shape[0]):
        assert list(ids[t]) == _brute_topk([float(v) for v in logits[t]], 5)
    assert list(ids[0][:3]) == [3, 7, 11]
    assert list(ids[1]) == [0, 1, 2, 3, 4]
    assert list(ids[3]) == [9, 0, 1, 2, 3]
    assert ids[4][0] == 2


def test_topk_weights_softmax_properties():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((20, 32)) * 3
    ids, w = O.route_from_logits(logits, 6, True)
    assert np.allclose(w.sum(1), 1.0, atol=1e-12)
    for t in range(20):
        l = logits[t, ids[t]]
        assert np.allclose(w[t] / w[t, 0], np.exp(l - l[0]), rtol=1e-12)
    ids2, w2 = O.route_from_logits(logits, 6, False)
    full = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    assert np.allclose(w2, np.take_along_axis(full, ids2.astype(np.int64), 1), rtol=1e-12)


def test_route_recomputes_near_ties_exactly():
    """Two experts whose exact logits differ below the float64 error bound, and
    two exactly equal experts: the certified route must follow exact order."""
    H, E, k = 64, 6, 3
    rng = np.random.default_rng(5)
    wr = (rng.standard_normal((H, E)) * 0.05).astype(np.float32)
    wr[:, 1] = wr[:, 4]                          # exact tie between 1 and 4
    x = synth.bf16_bits_from_f32(np.abs(rng.standard_normal((1, H))).astype(np.float32) + 1)
    xv = O.bf16_value(x)[0]
    # make expert 2 the best and 3 a hair above it (exactly one fp32 ulp of a
    # weight times x[0], far below the certification bound)
    wr[:, 2] += np.float32(0.5)
    wr[:, 3] = wr[:, 2]
    wr[0, 3] = np.nextafter(wr[0, 2], np.float32(np.inf))
    R = O.route(x, wr, None, k)
    assert R.recomputed[0]
    exact = [sum(Fraction(float(xv[h])) * Fraction(float(wr[h, e])) for h in range(H)) for e in range(E)]
    order = sorted(range(E), key=lambda e: (-exact[e], e))
    assert list(R.ids[0]) == order[:k]
    assert list(R.ids[0][:2]) == [3, 2]


# ---------------------------------------------------------------------------
# grouping
# ---------------------------------------------------------------------------
def test_permute_invariants_and_brute_force():
    rng = np.random.default_rng(6)
    T, k, E = 37, 4, 9
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    G = O.permute(ids, E)
    # brute force: buckets filled in (t, j) order
    buckets = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            buckets[ids[t, j]].append(t * k + j)
    assert list(G.counts) == [len(b) for b in buckets]
    assert list(G.offsets) == [0] + list(np.cumsum([len(b) for b in buckets]))
    assert list(G.perm_to_pair) == [p for b in buckets for p in b]
    assert np.array_equal(G.perm_to_pair[G.pair_to_perm], np.arange(T * k))
    tok = G.perm_to_pair // k
    assert np.array_equal(np.bincount(tok, minlength=T), np.full(T, k))   # each token k times


# ---------------------------------------------------------------------------
# expert FFN and combine
# ---------------------------------------------------------------------------
def _fsum_dot(a, b):
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def test_single_expert_layer_is_a_dense_swiglu_mlp():
    """E=1, k=1, no shared expert: the layer is a dense SwiGLU MLP; checked
    against plain Python loops with correctly rounded dot products."""
    w = synth.scaled(TINY, name="dense", T=3, H=64, E=1, I=32, top_k=1)
    L = synth.make_layer(w)
    x = synth.make_x(w)
    res = O.layer_forward(L, x)
    xv = O.bf16_value(x)
    Wg, Wu, Wd = (F.dequant(q, 0) for q in (L.gate, L.up, L.down))
    for t in range(w.T):
        h = []
        for i in range(w.I):
            g = _fsum_dot(xv[t], Wg[i])
            u = _fsum_dot(xv[t], Wu[i])
            a = g / (1 + math.exp(-g)) * u
            h.append(float(O.round_bf16(np.array([a]))[0]))
        assert np.allclose(res.h[t, 0], h, rtol=0, atol=0) or \
            np.max(np.abs(res.h[t, 0] - h) / (np.abs(h) + 1e-30)) <= 2.0 ** -7
        for n in range(w.H):
            yn = _fsum_dot(h, Wd[n])
            assert abs(res.out64[t, n] - yn) <= 1e-12 * (1 + abs(yn))
    assert np.all(res.routing.ids == 0) and np.all(res.routing.weights == 1.0)


def test_identical_experts_make_routing_irrelevant():
    w = synth.scaled(TINY, name="same", T=5, E=6, top_k=3)
    L = synth.make_layer(w)
    for q in (L.gate, L.up, L.down):
        q.codes[:] = q.codes[0]
        q.scales[:] = q.scales[0]
        q.tensor_scale[:] = q.tensor_scale[0]
    x = synth.make_x(w)
    res = O.layer_forward(L, x)
    ref = O.layer_forward(synth.LayerWeights(L.H, L.I, 1, 1, True, L.router_w[:, :1], None,
                                             *(synth.QWeight(q.fmt, q.rows, q.cols, 1, q.codes[:1],
                                                             q.scales[:1], q.tensor_scale[:1])
                                               for q in (L.gate, L.up, L.down))), x)
    assert np.allclose(res.out64, ref.out64, rtol=1e-13, atol=1e-15)


def test_down_tensor_scale_power_of_two_scales_output_exactly():
    L = synth.make_layer(TINY)
    x = synth.make_x(TINY)
    a = O.layer_forward(L, x)
    L.down.tensor_scale = L.down.tensor_scale * np.float32(8.0)
    b = O.layer_forward(L, x)
    assert np.array_equal(b.y, a.y * 8.0)
    assert np.array_equal(b.out64, a.out64 * 8.0)


def test_tiny_layer_end_to_end_vs_fsum_brute_force():
    """The whole tiny layer with every dot product correctly rounded."""
    L = synth.make_layer(TINY)
    x = synth.make_x(TINY)
    res = O.layer_forward(L, x)
    xv = O.bf16_value(x)
    for t in range(TINY.T):
        logits = [math.fsum([float(xv[t, h]) * float(L.router_w[h, e]) for h in range(TINY.H)])
                  for e in range(TINY.E)]
        sel = sorted(range(TINY.E), key=lambda e: (-logits[e], e))[:TINY.top_k]
        assert list(res.routing.ids[t]) == sel
        z = [math.exp(logits[e] - logits[sel[0]]) for e in sel]
        wts = [v / sum(z) for v in z]
        acc = [0.0] * TINY.H
        for j, e in enumerate(sel):
            Wg, Wu, Wd = (F.dequant(q, e) for q in (L.gate, L.up, L.down))
            h = []
            for i in range(TINY.I):
                g = _fsum_dot(xv[t], Wg[i])
                u = _fsum_dot(xv[t], Wu[i])
                h.append(float(O.round_bf16(np.array([g / (1 + math.exp(-g)) * u]))[0]))
            for n in range(TINY.H):
                acc[n] += wts[j] * _fsum_dot(h, Wd[n])
        assert np.allclose(res.out64[t], acc, rtol=1e-11, atol=1e-14)
        assert np.max(np.abs(res.out[t] - O.round_bf16(np.array(acc)))) <= \
            np.max(np.abs(acc)) * 2.0 ** -7


def test_route_from_table_hand_worked():
    """Token-table routing: experts from the table row of the token id, the
    weights the softmax of the selected logits (closed form)."""
    logits = np.array([[0.0, 1.0, 2.0, 3.0], [5.0, 4.0, 3.0, 2.0], [0.0, 0.0, 0.0, 0.0]])
    table = np.array([[3, 0], [1, 2], [2, 9]])  # row 2 holds an entry outside [0, E)
    ids, w = O.route_from_table([1, 0, 2], table, logits)
    assert ids.tolist() == [[1, 2], [3, 0], [2, 9]]
    e = np.exp(1.0)
    assert np.allclose(w[0], [1 / (1 + e), e / (1 + e)], rtol=1e-15)
    assert np.allclose(w[1], [1 / (1 + e ** 3), e ** 3 / (1 + e ** 3)], rtol=1e-15)  # logits 2, 5
    assert w[2].tolist() == [1.0, 0.0]
    ids, w = O.route_from_table([7, -1, 0], table, logits)   # token ids outside [0, V)
    assert ids[0].tolist() == [-1, -1] and ids[1].tolist() == [-1, -1] and np.all(w[:2] == 0)
    # full softmax gathered: weights sum to the selected share of the softmax
    ids, w = O.route_from_table([0], table, logits[:1], renormalize=False)
    z = np.exp(logits[0] - 3.0)
    assert np.allclose(w[0], z[[3, 0]] / z.sum(), rtol=1e-15)


def test_permute_drops_out_of_range_ids():
    """Pairs whose expert id is outside [0, E) are dropped: counted nowhere,
    placed after the sorted pairs, pair_to_perm -1; the rest is the stable
    sort of the valid pairs."""
    ids = np.array([[2, -1], [0, 5], [2, 0]], dtype=np.int32)   # E = 3
    G = O.permute(ids, 3)
    assert G.counts.tolist() == [2, 0, 2] and G.offsets.tolist() == [0, 2, 2, 4]
    assert G.perm_to_pair[:4].tolist() == [2, 5, 0, 4]
    assert G.pair_to_perm.tolist() == [2, -1, 0, -1, 3, 1]
    assert sorted(G.perm_to_pair[4:].tolist()) == [1, 3]
