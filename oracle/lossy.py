"""Opt-in lossy activation modes of the expert GEMMs — TEST INFRASTRUCTURE.

The default chain keeps activations in BF16.  The pages also name levers that
quantize the GEMM inputs so that low-precision matrix units can run them, each
explicit and off by default: NVFP4 W4A4 prefill, gated behind an opt-in switch
after first being on by default (forum thread "DGPP: a GB10-optimized C++/CUDA
inference engine", page 5, the update post; gitee "dgpp" README, "Execution
and performance", the NVFP4 W4A4 row), and an FP8 prefill GEMM with per-token
1x128 E4M3 activations against the checkpoint's 128x128 weight scales (same
README table, ``engine.prefill_fp8_gemm``, marked not bitwise).

The modes mirrored here, and the readings taken (the pages give no arithmetic
for any of them):

* ``"mxfp8"`` (W4A8, MXFP4 experts) and ``"mxfp4"`` (W4A4, MXFP4 experts):
  each GEMM input row is cut into blocks of 32 consecutive K and converted to
  an OCP MX block (OCP Microscaling Formats v1.0, the section on converting a
  vector of scalars to MX): shared exponent = floor(log2(max|v|)) minus the
  largest normal exponent of the element format (8 for E4M3, 2 for E2M1),
  clamped to the E8M0 range [-127, 127]; each element is v / 2^shared,
  clamped to the element format's largest magnitude and rounded to nearest,
  ties to even.  An all-zero block takes the smallest scale (code 0).  A
  block holding a non-finite value gets the NaN scale 0xFF and zero codes.
  MX block scales are 32 wide; the pages' W4A4 is NVFP4-shaped (16-wide E4M3
  scales), which the matrix units' E8M0-per-32 scale operand cannot carry,
  so the MX modes are offered for MXFP4 experts, whose weights already have
  that shape.
* ``"fp8_t128"`` (FP8 block-128 experts): each row is cut into blocks of 128
  K; per block s = fp32(max(max|v|, 2^-64) / 448) and each element is
  e4m3_RNE(clamp(fp32(v / s), -448, 448)), both divisions IEEE fp32.  A
  block holding a non-finite value gets s = NaN and zero codes.
* In every mode the GEMM input is the BF16 activation the exact chain would
  use (x for gate/up; the BF16 h = bf16(silu(g) * u) for down), quantized
  as above; the GEMM then contracts the dequantized values exactly.
* A mode applies to the projections whose weight format it names (MXFP4 for
  the MX modes, FP8 block-128 for ``fp8_t128``); every other projection runs
  the exact chain.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import formats
from . import layer as _layer

MODES = ("mxfp8", "mxfp4", "fp8_t128")

# element grids: every nonnegative magnitude with its code, in code order
_E4M3_CODES = np.arange(0x7F)                 # 0x00..0x7E (0x7F is NaN)
_E4M3_MAGS = formats.e4m3_value(_E4M3_CODES)  # increasing with the code
_E2M1_CODES = np.arange(8)
_E2M1_MAGS = formats.e2m1_value(_E2M1_CODES)

ELEM = {
    # name: (codes, magnitudes, largest normal exponent, sign bit)
    "e4m3": (_E4M3_CODES, _E4M3_MAGS, 8, 0x80),
    "e2m1": (_E2M1_CODES, _E2M1_MAGS, 2, 0x8),
}


def round_to_element(q, elem: str) -> np.ndarray:
    """Codes of the element-format values nearest to q (float64), ties to the
    even code (mantissa bit 0 clear); |q| beyond the largest value saturates.

    The search is a brute-force nearest over the format's value grid."""
    codes, mags, _, sbit = ELEM[elem]
    q = np.asarray(q, dtype=np.float64)
    a = np.minimum(np.abs(q), mags[-1])
    i = np.clip(np.searchsorted(mags, a), 1, len(mags) - 1)  # mags[i-1] < a <= mags[i] (or a == 0)
    lo, hi = mags[i - 1], mags[i]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((codes[i] & 1) == 0))
    c = np.where(pick_hi, codes[i], codes[i - 1]).astype(np.int64)
    c = np.where(a == 0, 0, c)
    c = np.where(np.signbit(q), c | sbit, c)
    return c.astype(np.uint8)


def mx_quantize(v, elem: str):
    """Rows of float64 values [..., K] (K % 32 == 0) -> (element codes
    uint8 [..., K], E8M0 scale codes uint8 [..., K/32])."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % 32 == 0
    _, mags, emax, _ = ELEM[elem]
    blk = v.reshape(v.shape[:-1] + (K // 32, 32))
    finite = np.all(np.isfinite(blk), axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(blk), blk, 0.0)), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    shared = np.where(amax > 0, e - emax, -127.0)
    shared = np.clip(shared, -127, 127)
    q = blk / np.exp2(shared)[..., None]
    codes = round_to_element(np.where(finite[..., None], q, 0.0), elem)
    codes = np.where(finite[..., None], codes, 0).astype(np.uint8)
    scales = np.where(finite, shared + 127, 255).astype(np.uint8)
    return codes.reshape(v.shape), scales


def mx_dequantize(codes, scales, elem: str) -> np.ndarray:
    codes = np.asarray(codes)
    dec = formats.e4m3_value if elem == "e4m3" else formats.e2m1_value
    K = codes.shape[-1]
    vals = dec(codes).reshape(codes.shape[:-1] + (K // 32, 32))
    return (vals * formats.e8m0_value(scales)[..., None]).reshape(codes.shape)


def t128_quantize(v):
    """Rows of bf16 values as float64 [..., K] -> (E4M3 codes uint8 [..., K],
    fp32 scales [..., ceil(K/128)]).  The last block may be shorter."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    nb = (K + 127) // 128
    codes = np.zeros(v.shape, dtype=np.uint8)
    scales = np.zeros(v.shape[:-1] + (nb,), dtype=np.float32)
    for b in range(nb):
        blk = v[..., 128 * b:min(K, 128 * b + 128)].astype(np.float32)  # bf16 -> fp32 exact
        finite = np.all(np.isfinite(blk), axis=-1)
        amax = np.max(np.abs(np.where(np.isfinite(blk), blk, np.float32(0))), axis=-1)
        amax = np.maximum(amax, np.float32(2.0 ** -64))
        s = (amax / np.float32(448.0)).astype(np.float32)       # IEEE fp32 division
        with np.errstate(invalid="ignore", over="ignore"):
            q = (blk / s[..., None]).astype(np.float32)         # IEEE fp32 division
        q = np.clip(q.astype(np.float64), -448.0, 448.0)
        c = round_to_element(np.where(finite[..., None], q, 0.0), "e4m3")
        codes[..., 128 * b:min(K, 128 * b + 128)] = np.where(finite[..., None], c, 0)
        scales[..., b] = np.where(finite, s, np.float32(np.nan))
    return codes, scales


def t128_dequantize(codes, scales) -> np.ndarray:
    codes = np.asarray(codes)
    K = codes.shape[-1]
    s = np.repeat(np.asarray(scales, dtype=np.float64), 128, axis=-1)[..., :K]
    return formats.e4m3_value(codes) * s


def mode_applies(mode: Optional[str], fmt: str) -> bool:
    """True when the mode quantizes the inputs of a projection in format fmt."""
    if mode is None:
        return False
    if mode in ("mxfp8", "mxfp4"):
        return fmt == "mxfp4"
    if mode == "fp8_t128":
        return fmt == "fp8_b128"
    raise ValueError(f"unknown mode {mode!r}")


def quantize_input(values, mode: str) -> np.ndarray:
    """The GEMM input as the mode's quantizer leaves it (float64 values)."""
    if mode == "mxfp8":
        return mx_dequantize(*mx_quantize(values, "e4m3"), "e4m3")
    if mode == "mxfp4":
        return mx_dequantize(*mx_quantize(values, "e2m1"), "e2m1")
    if mode == "fp8_t128":
        return t128_dequantize(*t128_quantize(values))
    raise ValueError(f"unknown mode {mode!r}")


def _input(values, mode, fmt):
    return quantize_input(values, mode) if mode_applies(mode, fmt) else values


def ffn(x64, wg, wu, wd, fmt_gu: str, fmt_d: str, mode: Optional[str]):
    """One expert's SwiGLU FFN on rows x64 with the mode's input quantization:
    h = bf16(silu(xq.Wg^T) * (xq.Wu^T)), y = hq.Wd^T (float64 contractions)."""
    xq = _input(x64, mode, fmt_gu)
    h = _layer.round_bf16(_layer.silu(xq @ wg.T) * (xq @ wu.T))
    hq = _input(h, mode, fmt_d)
    return h, hq @ wd.T


@dataclass
class LossyResult:
    routing: "_layer.Routing"
    tokens: np.ndarray
    h: np.ndarray
    y: np.ndarray
    y_shared: Optional[np.ndarray]
    out: np.ndarray
    out64: np.ndarray


def layer_forward(L, x_bits: np.ndarray, mode: Optional[str], tokens=None,
                  routing=None, decoded=None) -> LossyResult:
    """The layer with the mode applied to every expert projection it names.
    Routing, grouping and the combine are those of the exact chain."""
    T = x_bits.shape[0]
    k = L.top_k
    R = routing if routing is not None else _layer.route(x_bits, L.router_w, L.router_bias, k,
                                                         L.renormalize)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    dec = decoded if decoded is not None else _layer._Decoded(L)
    x64 = _layer.bf16_value(x_bits[toks])
    n = toks.size
    h = np.zeros((n, k, L.I))
    y = np.zeros((n, k, L.H))
    sel = R.ids[toks]
    for e in np.unique(sel):
        if not 0 <= e < L.E:  # a dropped pair: no FFN, y stays 0
            continue
        rows, slots = np.nonzero(sel == e)
        he, ye = ffn(x64[rows], dec("gate", int(e)), dec("up", int(e)), dec("down", int(e)),
                     L.gate.fmt, L.down.fmt, mode)
        h[rows, slots] = he
        y[rows, slots] = ye
    ys = None
    if L.has_shared:
        _, ys = ffn(x64, dec("sh_gate", 0), dec("sh_up", 0), dec("sh_down", 0),
                    L.sh_gate.fmt, L.sh_down.fmt, mode)
    out, out64 = _layer.combine(y, R.weights[toks], ys)
    return LossyResult(R, toks, h, y, ys, out, out64)
