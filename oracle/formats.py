"""Decoders for the stored weight formats, to float64 — TEST INFRASTRUCTURE.

Every decoder works from the bit fields of the code, as the format
specification defines them:

* E2M1 (OCP Microscaling Formats v1.0, FP4 element): 1 sign bit, 2 exponent
  bits (bias 1), 1 mantissa bit; exponent field 0 is subnormal (m * 0.5).
  No infinities or NaN.
* E4M3 "fn" (OCP 8-bit Floating Point, E4M3): 1 sign, 4 exponent (bias 7),
  3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the all-ones
  exponent with all-ones mantissa is NaN; there is no infinity.
* E8M0 (OCP Microscaling Formats v1.0, scale): 8-bit biased exponent
  (bias 127), value 2^(c-127); 0xFF is NaN.

Layouts of the checkpoint formats (the pages serve these as published, "DGPP"
README intro bullet on checkpoint formats; forum opening post, quantization
table):

* NVFP4: codes uint8 [rows][cols/2], the even K index in the low nibble;
  E4M3 scale per 16 consecutive K of a row, [rows][cols/16]; one fp32 tensor
  scale per expert tensor.  W[n,k] = e2m1(q[n,k]) * e4m3(S[n,k//16]) * ts.
* MXFP4: same codes, E8M0 scale per 32 K, [rows][cols/32].
  W[n,k] = e2m1(q[n,k]) * e8m0(S[n,k//32]).
* FP8 block-128: codes uint8 E4M3 [rows][cols]; fp32 scale per 128x128 block
  [ceil(rows/128)][ceil(cols/128)] (the checkpoint's 128x128 weight scales,
  gitee "dgpp" README, "Execution and performance", ``engine.prefill_fp8_gemm``).
  W[n,k] = e4m3(Q[n,k]) * S[n//128, k//128].
* MXFP8 (OCP MX v1.0 E4M3 elements): codes uint8 E4M3 [rows][cols], E8M0
  scale per 32 K, [rows][cols/32].  W[n,k] = e4m3(Q[n,k]) * e8m0(S[n,k//32]).
  The pages list MXFP8 among the formats read as published ("DGPP" README,
  intro bullet on checkpoint formats) and serve shared experts in it (README
  variant, supported-models table).
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code) -> np.ndarray:
    """E2M1 code (0..15) -> float64."""
    c = np.asarray(code).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def e4m3_value(code) -> np.ndarray:
    """E4M3 "fn" code (0..255) -> float64 (NaN for the two NaN codes)."""
    c = np.asarray(code).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e8m0_value(code) -> np.ndarray:
    """E8M0 code (0..255) -> float64 (NaN for 0xFF)."""
    c = np.asarray(code).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., n/2] -> codes [..., n]; even index from the low nibble."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, tensor_scale: float) -> np.ndarray:
    """One expert's NVFP4 matrix -> float64 [rows][cols]."""
    q = e2m1_value(unpack_nibbles(codes))
    s = e4m3_value(scales)
    return q * np.repeat(s, 16, axis=-1) * float(tensor_scale)


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's MXFP4 matrix -> float64 [rows][cols]."""
    q = e2m1_value(unpack_nibbles(codes))
    s = e8m0_value(scales)
    return q * np.repeat(s, 32, axis=-1)


def dequant_fp8_b128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's FP8 E4M3 block-128 matrix -> float64 [rows][cols]."""
    rows, cols = codes.shape
    q = e4m3_value(codes)
    s = np.asarray(scales, dtype=np.float64)
    s_full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:rows, :cols]
    return q * s_full


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's MXFP8 matrix -> float64 [rows][cols]."""
    q = e4m3_value(codes)
    s = e8m0_value(scales)
    return q * np.repeat(s, 32, axis=-1)


def dequant(qw, expert: int) -> np.ndarray:
    """Decode expert `expert` of a stored projection (any format)."""
    if qw.fmt == "nvfp4":
        return dequant_nvfp4(qw.codes[expert], qw.scales[expert], qw.tensor_scale[expert])
    if qw.fmt == "mxfp4":
        return dequant_mxfp4(qw.codes[expert], qw.scales[expert])
    if qw.fmt == "fp8_b128":
        return dequant_fp8_b128(qw.codes[expert], qw.scales[expert])
    if qw.fmt == "mxfp8":
        return dequant_mxfp8(qw.codes[expert], qw.scales[expert])
    raise ValueError(f"unknown format {qw.fmt!r}")
