"""Seeded synthetic inputs for the routed mixture-of-experts layer.

This module is the one place both the CPU oracle and the GPU path get their
inputs from.  It holds data containers, seeded random draws and the
*checkpoint encoders* that turn float weights into the stored formats (what a
checkpoint exporter does before any inference engine sees the weights).  It
holds no step of the layer itself: nothing here decodes a weight, computes a
logit, selects an expert, multiplies a matrix or combines a result.

Workload shapes follow the routed-expert formats the DGPP pages serve
("DGPP: a GB10-optimized C++/CUDA inference engine", opening post, the
quantization table: NVFP4 and MXFP4 routed experts, FP8 block-128 shared
experts, BF16 activations).  The value distributions are the synthetic ones
this library is measured on: activations ~N(0,1) rounded to bf16, router
weights ~N(0,0.05) in fp32, expert weights ~N(0,0.02) encoded to the stored
format, and optional Zipf(s=1.1) expert popularity offsets on the router.

Encoders (generator side only):

* NVFP4 (OCP MX-style E2M1 elements, one E4M3 scale per 16 elements along K,
  one fp32 tensor scale per expert tensor): ts = amax/(6*448);
  s_b = RNE_e4m3(amax_b/(6*ts)); q = RNE_e2m1(w/(s_b*ts)) saturated to +-6.
  Two codes per byte, the even K index in the low nibble.
* MXFP4 (OCP MX v1.0): E8M0 scale 2^X per 32 elements with
  X = floor(log2(amax_b)) - 2, q = RNE_e2m1(w/2^X) saturated to +-6.
* FP8 E4M3 ("fn", no infinities) with one fp32 scale per 128x128 block:
  s = amax_blk/448, q = RNE_e4m3(w/s).
* MXFP8 (OCP MX v1.0, E4M3 elements): E8M0 scale 2^X per 32 elements with
  X = floor(log2(amax_b)) - 8, q = RNE_e4m3(w/2^X) saturated to +-448.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GENERATOR_VERSION = 1

FMT_NVFP4 = "nvfp4"
FMT_MXFP4 = "mxfp4"
FMT_FP8 = "fp8_b128"
FMT_MXFP8 = "mxfp8"
FORMATS = (FMT_NVFP4, FMT_MXFP4, FMT_FP8, FMT_MXFP8)

# Sub-seed identifiers: every tensor draws from SeedSequence(seed, (id, expert)).
_TID = {"x": 1, "router": 2, "zipf_perm": 3, "gate": 4, "up": 5, "down": 6,
        "sh_gate": 7, "sh_up": 8, "sh_down": 9}


# --------------------------------------------------------------------------
# containers
# --------------------------------------------------------------------------
@dataclass
class QWeight:
    """One projection of E stacked experts, logical [rows=out][cols=in]."""
    fmt: str
    rows: int
    cols: int
    num_experts: int
    codes: np.ndarray                 # uint8 [E][rows][cols/2] (fp4) or [E][rows][cols] (fp8)
    scales: np.ndarray                # uint8 e4m3 [E][rows][cols/16] | uint8 e8m0 [E][rows][cols/32]
                                      # | float32 [E][ceil(rows/128)][ceil(cols/128)]
    tensor_scale: Optional[np.ndarray] = None   # float32 [E] (NVFP4 only)

    def nbytes_per_expert(self) -> int:
        n = self.codes[0].nbytes + self.scales[0].nbytes
        if self.tensor_scale is not None:
            n += 4
        return n


@dataclass
class LayerWeights:
    H: int
    I: int
    E: int
    top_k: int
    renormalize: bool
    router_w: np.ndarray               # float32 [H][E]
    router_bias: Optional[np.ndarray]  # float32 [E] or None
    gate: QWeight
    up: QWeight
    down: QWeight
    I_shared: int = 0
    sh_gate: Optional[QWeight] = None
    sh_up: Optional[QWeight] = None
    sh_down: Optional[QWeight] = None

    @property
    def has_shared(self) -> bool:
        return self.sh_gate is not None


@dataclass(frozen=True)
class Workload:
    """A named workload: shapes, formats and input recipe."""
    name: str
    T: int
    H: int
    E: int
    I: int
    top_k: int
    fmt: str
    I_shared: int = 0
    shared_fmt: Optional[str] = None
    # down projections in another format than gate/up (None: the same)
    down_fmt: Optional[str] = None
    shared_down_fmt: Optional[str] = None
    zipf_s: Optional[float] = None
    weight_sets: int = 1
    renormalize: bool = True
    x_std: float = 1.0
    router_std: float = 0.05
    w_std: float = 0.02
    seed: int = 0
    note: str = ""


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_nvfp4_t4", T=4, H=256, E=8, I=128, top_k=2, fmt=FMT_NVFP4,
                 note="tiny layer, no shared expert"),
        Workload("decode_t1_nvfp4", T=1, H=2048, E=512, I=512, top_k=10, fmt=FMT_NVFP4,
                 I_shared=512, shared_fmt=FMT_FP8, weight_sets=48,
                 note="single-sequence decode, 48 cycled layer weight sets"),
        Workload("decode_t8_nvfp4_zipf", T=8, H=2048, E=512, I=512, top_k=10, fmt=FMT_NVFP4,
                 I_shared=512, shared_fmt=FMT_FP8, zipf_s=1.1, weight_sets=48,
                 note="8 concurrent sequences, Zipf expert popularity"),
        Workload("decode_t8_mxfp4_zipf", T=8, H=2048, E=512, I=512, top_k=10, fmt=FMT_MXFP4,
                 I_shared=512, shared_fmt=FMT_FP8, zipf_s=1.1, weight_sets=48,
                 note="8 concurrent sequences, MXFP4 routed experts"),
        Workload("decode_t32_nvfp4_zipf", T=32, H=2048, E=512, I=512, top_k=10, fmt=FMT_NVFP4,
                 I_shared=512, shared_fmt=FMT_FP8, zipf_s=1.1, weight_sets=48,
                 note="32 rows (batched decode / speculative verify), Zipf expert popularity"),
        Workload("decode_t64_nvfp4_zipf", T=64, H=2048, E=512, I=512, top_k=10, fmt=FMT_NVFP4,
                 I_shared=512, shared_fmt=FMT_FP8, zipf_s=1.1, weight_sets=48,
                 note="64 rows (batched decode / speculative verify), Zipf expert popularity"),
        Workload("decode_t8_fp8_wide", T=8, H=6144, E=256, I=2048, top_k=8, fmt=FMT_FP8,
                 I_shared=2048, shared_fmt=FMT_FP8, weight_sets=8,
                 note="wide FP8 block-128 experts, 8 cycled layer weight sets"),
        Workload("prefill_t8192_mxfp4_zipf", T=8192, H=2048, E=512, I=512, top_k=10,
                 fmt=FMT_MXFP4, I_shared=512, shared_fmt=FMT_FP8, zipf_s=1.1,
                 note="prefill chunk, MXFP4 routed experts, uneven expert groups"),
        Workload("prefill_t8192_fp8_wide", T=8192, H=6144, E=256, I=2048, top_k=8,
                 fmt=FMT_FP8, I_shared=2048, shared_fmt=FMT_FP8,
                 note="prefill chunk, wide FP8 block-128 experts"),
        Workload("prefill_t8192_nvfp4_zipf", T=8192, H=2048, E=512, I=512, top_k=10,
                 fmt=FMT_NVFP4, I_shared=512, shared_fmt=FMT_FP8, zipf_s=1.1,
                 note="prefill chunk, uneven expert groups"),
    ]
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (used for small test cases)."""
    d = dict(w.__dict__)
    d.update(changes)
    return Workload(**d)


# --------------------------------------------------------------------------
# seeded draws
# --------------------------------------------------------------------------
def _rng(seed: int, tensor: str, expert: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(_TID[tensor], expert))
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def make_x(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Activations: bf16 bits [T][H], values N(0, x_std) rounded to bf16."""
    T = w.T if T is None else T
    g = _rng(w.seed, "x")
    a = g.standard_normal((T, w.H), dtype=np.float32) * np.float32(w.x_std)
    return bf16_bits_from_f32(a)


def make_router(w: Workload):
    g = _rng(w.seed, "router")
    wr = (g.standard_normal((w.H, w.E), dtype=np.float32) * np.float32(w.router_std))
    bias = None
    if w.zipf_s is not None:
        # Expert popularity ranks r = 1 + a seeded permutation of 0..E-1.  An
        # offset of -s*ln(r), scaled from Gumbel units to the std of the
        # router logits (router_std*x_std*sqrt(H)), gives Zipf(s) popularity
        # under Gaussian logit noise.
        perm = _rng(w.seed, "zipf_perm").permutation(w.E)
        r = 1.0 + perm.astype(np.float64)
        sigma_l = w.router_std * w.x_std * math.sqrt(w.H)
        sigma_g = math.pi / math.sqrt(6.0)
        bias = (-w.zipf_s * np.log(r) * sigma_l / sigma_g).astype(np.float32)
    return wr, bias


# --------------------------------------------------------------------------
# checkpoint encoders
# --------------------------------------------------------------------------
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2.0


def enc_e2m1(v: np.ndarray) -> np.ndarray:
    """float -> 4-bit E2M1 codes (RNE, saturating at 6); sign in bit 3.

    The magnitude code counts the grid midpoints below |v|; a value exactly on
    a midpoint goes to the even code."""
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.uint8)
    for i, m in enumerate(_E2M1_MID):
        code += a > m
        if i % 2 == 1:              # midpoint between odd code i and even code i+1
            code += a == m
    neg = (v < 0) & (code != 0)
    return code | (neg.astype(np.uint8) << 3)


def round_e4m3(v: np.ndarray):
    """float -> (E4M3 "fn" code, the rounded value), RNE, saturating at +-448.

    The value is the rounding result itself (mantissa and exponent chosen by
    the rounding), which the exporter needs to divide the weights by."""
    v = v.astype(np.float64)
    a = np.minimum(np.abs(v), 448.0)
    f, ex = np.frexp(a)                       # a = f*2^ex, f in [0.5,1)
    e = ex - 1                                # a = (2f)*2^e
    normal = a >= 2.0 ** -6
    mq_n = np.rint((2.0 * f - 1.0) * 8.0)     # 3-bit mantissa, ties to even
    e_n = np.where(mq_n == 8, e + 1, e)
    mq_n = np.where(mq_n == 8, 0, mq_n)
    code_n = ((e_n + 7) << 3) + mq_n
    val_n = (1.0 + mq_n / 8.0) * np.exp2(e_n.astype(np.float64))
    mq_s = np.rint(a / 2.0 ** -9)             # subnormal: m * 2^-9 (8 -> min normal)
    code = np.where(normal, code_n, mq_s).astype(np.int64)
    val = np.where(normal, val_n, mq_s * 2.0 ** -9)
    code = np.clip(code, 0, 0x7E).astype(np.uint8)
    neg = (v < 0) & (code != 0)
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8), np.where(neg, -val, val)


def enc_e4m3(v: np.ndarray) -> np.ndarray:
    return round_e4m3(v)[0]


def _pack_nibbles(c: np.ndarray) -> np.ndarray:
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def encode_nvfp4(w: np.ndarray):
    rows, cols = w.shape
    assert cols % 16 == 0
    w = w.astype(np.float64)
    amax = float(np.max(np.abs(w))) if w.size else 0.0
    ts = np.float32(amax / (6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    blk = w.reshape(rows, cols // 16, 16)
    amax_b = np.max(np.abs(blk), axis=2)
    sc, sval = round_e4m3(amax_b / (6.0 * float(ts)))
    sv = sval * float(ts)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sv[..., None] > 0, blk / sv[..., None], 0.0)
    codes = enc_e2m1(q).reshape(rows, cols)
    return _pack_nibbles(codes), sc, ts


def encode_mxfp4(w: np.ndarray):
    rows, cols = w.shape
    assert cols % 32 == 0
    w = w.astype(np.float64)
    blk = w.reshape(rows, cols // 32, 32)
    amax_b = np.max(np.abs(blk), axis=2)
    with np.errstate(divide="ignore"):
        X = np.where(amax_b > 0, np.floor(np.log2(np.where(amax_b > 0, amax_b, 1.0))) - 2, -127)
    X = np.clip(X, -127, 127)
    q = blk / np.exp2(X)[..., None]
    codes = enc_e2m1(q).reshape(rows, cols)
    return _pack_nibbles(codes), (X + 127).astype(np.uint8)


def encode_fp8_b128(w: np.ndarray):
    rows, cols = w.shape
    rb, cb = -(-rows // 128), -(-cols // 128)
    w = w.astype(np.float64)
    s = np.zeros((rb, cb), dtype=np.float32)
    q = np.zeros((rows, cols), dtype=np.uint8)
    for i in range(rb):
        for j in range(cb):
            b = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            amax = float(np.max(np.abs(b)))
            sj = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
            s[i, j] = sj
            q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128] = enc_e4m3(b / float(sj))
    return q, s


def encode_mxfp8(w: np.ndarray):
    rows, cols = w.shape
    assert cols % 32 == 0
    w = w.astype(np.float64)
    blk = w.reshape(rows, cols // 32, 32)
    amax_b = np.max(np.abs(blk), axis=2)
    with np.errstate(divide="ignore"):
        X = np.where(amax_b > 0, np.floor(np.log2(np.where(amax_b > 0, amax_b, 1.0))) - 8, -127)
    X = np.clip(X, -127, 127)
    q = blk / np.exp2(X)[..., None]
    return enc_e4m3(q).reshape(rows, cols), (X + 127).astype(np.uint8)


def _gen_matrix(args):
    seed, tensor, expert, rows, cols, fmt, std = args
    g = _rng(seed, tensor, expert)
    w = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    if fmt == FMT_NVFP4:
        c, s, ts = encode_nvfp4(w)
        return c, s, ts
    if fmt == FMT_MXFP4:
        c, s = encode_mxfp4(w)
        return c, s, None
    if fmt == FMT_FP8:
        c, s = encode_fp8_b128(w)
        return c, s, None
    if fmt == FMT_MXFP8:
        c, s = encode_mxfp8(w)
        return c, s, None
    raise ValueError(fmt)


def make_qweight(seed: int, tensor: str, E: int, rows: int, cols: int, fmt: str,
                 std: float, pool: Optional[ProcessPoolExecutor] = None) -> QWeight:
    jobs = [(seed, tensor, e, rows, cols, fmt, std) for e in range(E)]
    res = list(pool.map(_gen_matrix, jobs, chunksize=max(1, E // 64))) if pool else \
        [_gen_matrix(j) for j in jobs]
    codes = np.stack([r[0] for r in res])
    scales = np.stack([r[1] for r in res])
    ts = np.array([r[2] for r in res], dtype=np.float32) if fmt == FMT_NVFP4 else None
    return QWeight(fmt, rows, cols, E, codes, scales, ts)


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_layer(w: Workload, workers: Optional[int] = None) -> LayerWeights:
    """All weights of one layer for workload `w` (deterministic in w.seed)."""
    wr, bias = make_router(w)
    n = default_workers() if workers is None else workers
    big = w.E * w.I * w.H >= (1 << 22)
    pool = None
    if n > 1 and big:
        import multiprocessing as mp
        pool = ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"))
    def note(what):  # progress of the long generations, on stderr
        if big:
            import sys
            print(f"[synth] {w.name}: {what} generated", file=sys.stderr, flush=True)

    try:
        gate = make_qweight(w.seed, "gate", w.E, w.I, w.H, w.fmt, w.w_std, pool)
        note("gate")
        up = make_qweight(w.seed, "up", w.E, w.I, w.H, w.fmt, w.w_std, pool)
        note("up")
        down = make_qweight(w.seed, "down", w.E, w.H, w.I, w.down_fmt or w.fmt, w.w_std, pool)
        note("down")
        sh = (None, None, None)
        if w.I_shared:
            sf = w.shared_fmt
            sh = (make_qweight(w.seed, "sh_gate", 1, w.I_shared, w.H, sf, w.w_std, pool),
                  make_qweight(w.seed, "sh_up", 1, w.I_shared, w.H, sf, w.w_std, pool),
                  make_qweight(w.seed, "sh_down", 1, w.H, w.I_shared, w.shared_down_fmt or sf,
                               w.w_std, pool))
    finally:
        if pool is not None:
            pool.shutdown()
    return LayerWeights(w.H, w.I, w.E, w.top_k, w.renormalize, wr, bias, gate, up, down,
                        w.I_shared, *sh)


def layer_bytes(L: LayerWeights) -> int:
    """Stored bytes of one layer weight set (all experts, router)."""
    n = L.router_w.nbytes + (L.router_bias.nbytes if L.router_bias is not None else 0)
    for q in (L.gate, L.up, L.down, L.sh_gate, L.sh_up, L.sh_down):
        if q is not None:
            n += q.codes.nbytes + q.scales.nbytes + (q.tensor_scale.nbytes if q.tensor_scale is not None else 0)
    return n
