"""The routed mixture-of-experts layer in float64 — TEST INFRASTRUCTURE.

Steps, in the order the layer runs them (the pages name the layer and list
per-format GEMV and GEMM kernels for it — "DGPP" README, source layout — but
print none of its arithmetic; where they are silent the reading taken is
stated here):

1. router logits  l[t,e] = sum_h x[t,h] * Wr[h,e] + b[e]   (x bf16, Wr fp32
   [H][E], b an optional per-expert logit offset).  Routing is decided on the
   exact logit rounded once to float64.  The products are exact in float64;
   the sum is taken by BLAS and certified with a rigorous error bound, and
   any token whose top-(k+1) order the bound cannot certify is recomputed
   with a correctly rounded sum (math.fsum).
2. top-k: order experts by (larger logit first, then lower expert id; NaN
   after every number); keep the first k, in that order.
3. weights: softmax over the k selected logits (renormalised), or the full
   softmax over all E gathered at the selected ids.
4. grouping: a stable counting sort of the pairs (t, j), t-major, keyed by
   expert; offsets are the exclusive scan of the counts.
5. expert FFN (SwiGLU): g = x.Wg^T, u = x.Wu^T, h = bf16_RNE(silu(g) * u);
   y = h.Wd^T.  The intermediate h is BF16 because activations stay BF16
   (forum thread "DGPP: a GB10-optimized C++/CUDA inference engine", opening
   post: "Activations stay BF16").
6. shared expert: the same FFN on every token with its own weights, weight 1.
7. combine: out[t] = bf16_RNE( sum_j w[t,j] * y[t,j]  +  y_shared[t] ), the
   per-expert partials kept in full precision and summed in slot order (the
   default chain sums expert partials in fp32; bf16 partials are an explicit
   lever — gitee "dgpp" README, "Execution and performance",
   ``engine.prefill_bf16_partials``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from functools import lru_cache
from typing import Optional

import numpy as np

from . import formats

_U64 = 2.0 ** -53


# ---------------------------------------------------------------------------
# bf16 values and rounding
# ---------------------------------------------------------------------------
def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(v) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits; the quantum of a value with leading
    bit 2^e is 2^(e-7), and 2^-133 below the normal range.  Values at or
    beyond the overflow midpoint become infinite; NaN stays NaN."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    fin = np.isfinite(a) & (a > 0)
    f, ex = np.frexp(np.where(fin, a, 1.0))          # a = f * 2^ex, f in [0.5, 1)
    q = np.exp2(np.maximum(ex - 8, -133).astype(np.float64))
    r = np.rint(np.where(fin, a, 0.0) / q) * q       # rint: ties to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(fin, r, a)                          # 0, inf, nan unchanged
    return np.copysign(r, v)


def bf16_bits(v) -> np.ndarray:
    """float64 values that are bf16-representable -> their uint16 bits."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------
def _gamma(n: int) -> float:
    return n * _U64 / (1.0 - n * _U64)


def router_logits(x_bits: np.ndarray, router_w: np.ndarray, bias: Optional[np.ndarray]):
    """float64 logits [T][E] and a rigorous per-token error bound [T].

    Every product bf16 x fp32 is exact in float64 (8 + 24 significant bits);
    any order of summing H+1 terms errs by at most gamma(H+1) * sum|terms|."""
    x = bf16_value(x_bits)
    w = np.asarray(router_w, dtype=np.float64)
    l = x @ w
    a = np.abs(x) @ np.abs(w)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        l = l + b
        a = a + np.abs(b)
    H = w.shape[0]
    # 2x slack covers the rounding in computing `a` itself.
    bound = 2.0 * _gamma(H + 2) * np.max(a, axis=1) if a.size else np.zeros(x.shape[0])
    return l, bound


def exact_logits_row(x_row_bits: np.ndarray, router_w: np.ndarray, bias) -> np.ndarray:
    """One token's logits, each the correctly rounded float64 of the exact sum."""
    x = bf16_value(x_row_bits)
    w = np.asarray(router_w, dtype=np.float64)
    E = w.shape[1]
    out = np.empty(E)
    for e in range(E):
        terms = x * w[:, e]
        if bias is not None:
            terms = np.append(terms, float(bias[e]))
        if np.all(np.isfinite(terms)):
            out[e] = math.fsum(terms.tolist())
        else:   # inf/nan: the IEEE result does not depend on the order
            out[e] = float(np.sum(terms))
    return out


def expert_order(l_row: np.ndarray) -> np.ndarray:
    """Expert ids sorted by (non-NaN first, larger logit first, lower id first)."""
    l_row = np.asarray(l_row, dtype=np.float64)
    nan = np.isnan(l_row)
    key = np.where(nan, 0.0, -l_row)
    ids = np.arange(l_row.shape[0])
    return np.lexsort((ids, key, nan))


def _certified(l_row: np.ndarray, order: np.ndarray, k: int, bound: float) -> bool:
    """True when every adjacent gap among the top min(k+1,E) exceeds 2*bound,
    which fixes the exact top-k set and its order."""
    top = l_row[order[:k + 1]]
    if not np.all(np.isfinite(top)):
        return False
    gaps = top[:-1] - top[1:]
    return bool(np.all(gaps > 2.0 * bound))


def topk_weights(l_sel: np.ndarray, l_all: Optional[np.ndarray], renormalize: bool) -> np.ndarray:
    """Routing weights for the selected logits (in selection order)."""
    l_sel = np.asarray(l_sel, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        if renormalize:
            z = np.exp(l_sel - l_sel[0])
            return z / np.sum(z)
        m = np.max(l_all)
        return np.exp(l_sel - m) / np.sum(np.exp(l_all - m))


@dataclass
class Routing:
    logits: np.ndarray      # float64 [T][E] (the values routing was decided on)
    ids: np.ndarray         # int32 [T][k]
    weights: np.ndarray     # float64 [T][k]
    recomputed: np.ndarray  # bool [T]: token needed the correctly rounded recompute
    bound: np.ndarray       # float64 [T]


def route(x_bits, router_w, bias, k: int, renormalize: bool = True) -> Routing:
    """Router softmax + top-k from activations (steps 1-3)."""
    l, bound = router_logits(x_bits, router_w, bias)
    T, E = l.shape
    ids = np.zeros((T, k), dtype=np.int32)
    wts = np.zeros((T, k))
    rec = np.zeros(T, dtype=bool)
    for t in range(T):
        order = expert_order(l[t])
        if not _certified(l[t], order, k, bound[t]):
            l[t] = exact_logits_row(x_bits[t], router_w, bias)
            order = expert_order(l[t])
            rec[t] = True
        ids[t] = order[:k]
        wts[t] = topk_weights(l[t, order[:k]], l[t], renormalize)
    return Routing(l, ids, wts, rec, bound)


def route_from_logits(logits: np.ndarray, k: int, renormalize: bool = True):
    """Top-k and weights on given logits (taken exactly as given)."""
    l = np.asarray(logits, dtype=np.float64)
    T = l.shape[0]
    ids = np.zeros((T, k), dtype=np.int32)
    wts = np.zeros((T, k))
    for t in range(T):
        order = expert_order(l[t])
        ids[t] = order[:k]
        wts[t] = topk_weights(l[t, order[:k]], l[t], renormalize)
    return ids, wts


def route_from_table(token_ids, table, logits, renormalize: bool = True):
    """Token-table routing: the experts of token t are row token_ids[t] of
    `table` [V][k], in table order; the weights are the layer's softmax (over
    the k selected logits, or the full softmax gathered) at those experts.
    The pages route the first layers of one served model by a token table
    and say no more; this is the plain reading (expert choice from the
    table, weighting by the layer's own router function).  A token id outside
    [0, V) selects nothing (ids -1, weights 0); a table entry outside [0, E)
    gets weight 0 and takes no part in the normalisation."""
    token_ids = np.asarray(token_ids, dtype=np.int64)
    table = np.asarray(table, dtype=np.int64)
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    V, k = table.shape
    ids = np.full((T, k), -1, dtype=np.int32)
    wts = np.zeros((T, k))
    for t in range(T):
        if not 0 <= token_ids[t] < V:
            continue
        row = table[token_ids[t]]
        ids[t] = row
        ok = (row >= 0) & (row < E)
        if not ok.any():
            continue
        sel = l[t, row[ok]]
        with np.errstate(invalid="ignore", over="ignore"):
            if renormalize:
                z = np.exp(sel - np.max(sel))
                wts[t, ok] = z / np.sum(z)
            else:
                m = np.max(l[t])
                wts[t, ok] = np.exp(sel - m) / np.sum(np.exp(l[t] - m))
    return ids, wts


# ---------------------------------------------------------------------------
# grouping
# ---------------------------------------------------------------------------
@dataclass
class Grouping:
    counts: np.ndarray        # int32 [E]
    offsets: np.ndarray       # int32 [E+1]
    perm_to_pair: np.ndarray  # int32 [T*k]: permuted row -> pair t*k+j
    pair_to_perm: np.ndarray  # int32 [T*k]: pair -> permuted row


def permute(ids: np.ndarray, E: int) -> Grouping:
    """Stable counting sort of the pairs (t, j), t-major, keyed by expert id.
    Pairs whose id is outside [0, E) are dropped: they follow the sorted pairs
    in perm_to_pair and have pair_to_perm -1."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    key = np.where(valid, flat, E)
    p2pair = np.argsort(key, kind="stable").astype(np.int32)
    pair2p = np.empty_like(p2pair)
    pair2p[p2pair] = np.arange(flat.size, dtype=np.int32)
    pair2p[~valid] = -1
    return Grouping(counts, offsets, p2pair, pair2p)


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------
def ffn_gate_up(x64: np.ndarray, wg: np.ndarray, wu: np.ndarray) -> np.ndarray:
    """h = bf16_RNE(silu(x.Wg^T) * (x.Wu^T)) for rows of x (float64 in, bf16 values out)."""
    g = x64 @ wg.T
    u = x64 @ wu.T
    return round_bf16(silu(g) * u)


def ffn_down(h64: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """y = h.Wd^T in float64."""
    return h64 @ wd.T


def combine(y_pairs: np.ndarray, w: np.ndarray, y_shared: Optional[np.ndarray]):
    """out[t] = bf16_RNE(sum_j w[t,j]*y[t,j] + y_shared[t]) summed in slot order.

    Returns (bf16 values as float64, the unrounded float64 sum)."""
    T, k, H = y_pairs.shape
    acc = np.zeros((T, H))
    for j in range(k):
        acc = acc + w[:, j:j + 1] * y_pairs[:, j, :]
    if y_shared is not None:
        acc = acc + y_shared
    return round_bf16(acc), acc


class _Decoded:
    """Per-expert decoded weights, decoded on first use."""

    def __init__(self, L, maxsize: int = 64):
        self.L = L
        self._get = lru_cache(maxsize=maxsize)(self._decode)

    def _decode(self, which: str, e: int) -> np.ndarray:
        return formats.dequant(getattr(self.L, which), e)

    def __call__(self, which: str, e: int) -> np.ndarray:
        return self._get(which, e)


@dataclass
class LayerResult:
    routing: Routing
    grouping: Grouping
    tokens: np.ndarray           # int [n] tokens whose FFN outputs were computed
    h: np.ndarray                # float64 [n][k][I]    (bf16 values)
    y: np.ndarray                # float64 [n][k][H]
    h_shared: Optional[np.ndarray]  # [n][I_s] (bf16 values)
    y_shared: Optional[np.ndarray]  # [n][H]
    out: np.ndarray              # float64 [n][H] (bf16 values)
    out64: np.ndarray            # float64 [n][H] before the final rounding


def layer_forward(L, x_bits: np.ndarray, tokens=None, routing: Optional[Routing] = None,
                  decoded: Optional[_Decoded] = None) -> LayerResult:
    """The whole layer.  Routing and grouping cover every token; the expert
    FFNs and the combine are evaluated for `tokens` (default: all)."""
    T = x_bits.shape[0]
    k = L.top_k
    R = routing if routing is not None else route(x_bits, L.router_w, L.router_bias, k, L.renormalize)
    G = permute(R.ids, L.E)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    dec = decoded if decoded is not None else _Decoded(L)
    x64 = bf16_value(x_bits[toks])
    n = toks.size
    h = np.zeros((n, k, L.I))
    y = np.zeros((n, k, L.H))
    sel = R.ids[toks]
    for e in np.unique(sel):
        if not 0 <= e < L.E:  # a dropped pair: no FFN, y stays 0
            continue
        rows, slots = np.nonzero(sel == e)
        he = ffn_gate_up(x64[rows], dec("gate", int(e)), dec("up", int(e)))
        h[rows, slots] = he
        y[rows, slots] = ffn_down(he, dec("down", int(e)))
    hs = ys = None
    if L.has_shared:
        hs = ffn_gate_up(x64, dec("sh_gate", 0), dec("sh_up", 0))
        ys = ffn_down(hs, dec("sh_down", 0))
    out, out64 = combine(y, R.weights[toks], ys)
    return LayerResult(R, G, toks, h, y, hs, ys, out, out64)
