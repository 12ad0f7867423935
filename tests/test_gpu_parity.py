"""GPU parity: the HIP path through the C ABI against the CPU oracle."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import layer as O

from gpu_util import assert_close, check_layer_against_oracle, device_layer, layer_for, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts too
    pytest.skip("no GPU", allow_module_level=True)

import quantized_moe_expert_02_amd as moe  # noqa: E402
from quantized_moe_expert_02_amd.device import bf16_bits, bf16_tensor  # noqa: E402

W = synth.WORKLOADS

# Small layers that still span several tiles, with ragged K chunks and row tiles.
SMALL = {
    "nvfp4_ragged": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_ragged", T=5, H=352, E=24, I=160,
                                 top_k=3, I_shared=96, shared_fmt=synth.FMT_FP8),
    "mxfp4_ragged": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_ragged", T=7, H=416, E=20, I=224,
                                 top_k=4, fmt=synth.FMT_MXFP4, I_shared=64,
                                 shared_fmt=synth.FMT_NVFP4, zipf_s=1.1),
    "fp8_ragged": synth.scaled(W["tiny_nvfp4_t4"], name="fp8_ragged", T=8, H=336, E=12, I=144,
                               top_k=2, fmt=synth.FMT_FP8, I_shared=272, shared_fmt=synth.FMT_FP8),
    "nvfp4_t3_k1": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_t3_k1", T=3, H=256, E=4, I=128,
                                top_k=1),
    # above the fused decode size, at most one GEMV pass per group
    "nvfp4_t12": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_t12", T=12, H=288, E=8, I=96,
                              top_k=3, I_shared=64, shared_fmt=synth.FMT_MXFP4),
    # K a multiple of 128 (FP4 block scales read by whole chunk): 8 and 3
    # chunks (the last batch of the down projection is partial)
    "nvfp4_aligned": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_aligned", T=6, H=1024, E=12,
                                  I=384, top_k=3, I_shared=128, shared_fmt=synth.FMT_NVFP4),
    "mxfp4_aligned": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_aligned", T=11, H=768, E=10,
                                  I=256, top_k=2, fmt=synth.FMT_MXFP4, I_shared=256,
                                  shared_fmt=synth.FMT_MXFP4, zipf_s=1.1),
    # K a multiple of 2048: the decode's aligned FP4 gate/up tile (K quarters
    # of one and of two four-chunk batches)
    "nvfp4_k2048": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_k2048", T=6, H=2048, E=12, I=256,
                                top_k=3, I_shared=128, shared_fmt=synth.FMT_NVFP4, zipf_s=1.1),
    "mxfp4_k4096": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_k4096", T=8, H=4096, E=10, I=128,
                                top_k=2, fmt=synth.FMT_MXFP4, I_shared=64,
                                shared_fmt=synth.FMT_FP8, zipf_s=1.1),
}


# Layers with T > 16 (tiled grouped GEMM): expert groups span several
# 128-row tiles, with ragged row tails, column tails (I, H not multiples of
# the 64/128-wide column tiles) and K tails (H, I not multiples of 64).
MID = {
    "nvfp4_mid": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_mid", T=300, H=352, E=6, I=160,
                              top_k=3, I_shared=96, shared_fmt=synth.FMT_FP8),
    "mxfp4_mid": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_mid", T=200, H=416, E=5, I=224,
                              top_k=2, fmt=synth.FMT_MXFP4, I_shared=64,
                              shared_fmt=synth.FMT_NVFP4, zipf_s=1.1),
    "fp8_mid": synth.scaled(W["tiny_nvfp4_t4"], name="fp8_mid", T=260, H=336, E=4, I=144,
                            top_k=2, fmt=synth.FMT_FP8, I_shared=272, shared_fmt=synth.FMT_FP8),
}


@pytest.mark.parametrize("name", ["tiny_nvfp4_t4"] + list(SMALL))
def test_layer_small(name):
    w = W.get(name) or SMALL[name]
    say(f"[gpu] layer {name}: T={w.T} H={w.H} E={w.E} I={w.I} k={w.top_k} fmt={w.fmt}")
    r = check_layer_against_oracle(layer_for(w), synth.make_x(w), what=name)
    say(f"[gpu] layer {name}: rel={r['rel']:.2e} worst={r['worst']:.2e}")


@pytest.mark.parametrize("name", ["decode_t1_nvfp4", "decode_t8_nvfp4_zipf", "decode_t8_mxfp4_zipf"])
def test_layer_decode_full(name):
    w = W[name]
    say(f"[gpu] layer {name} (full size)")
    r = check_layer_against_oracle(layer_for(w), synth.make_x(w), what=name)
    say(f"[gpu] layer {name}: rel={r['rel']:.2e} worst={r['worst']:.2e} "
        f"unique experts={len(np.unique(r['ids']))}")


# 9 to 32 rows with the aligned (lean) tiles in every launch: the decode
# lowering (decode router, block top-k, per-group gate/up, per-expert down,
# combine); expert groups go through the MFMA B operand's 16 columns in
# chunks of 16 rows, and more than 256 pair slots take two rounds of the
# group derivation.
DECODE_ROWS = {
    # k = E: every group holds all 16 tokens
    "nvfp4_t16_full_groups": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_t16_full_groups", T=16,
                                          H=2048, E=4, I=512, top_k=4, I_shared=512,
                                          shared_fmt=synth.FMT_NVFP4),
    "mxfp4_t9_k4096": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_t9_k4096", T=9, H=4096, E=10,
                                   I=512, top_k=2, fmt=synth.FMT_MXFP4, I_shared=1024,
                                   shared_fmt=synth.FMT_FP8, zipf_s=1.1),
    "nvfp4_t13_fp8_down": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_t13_fp8_down", T=13,
                                       H=2048, E=12, I=1024, top_k=3, fmt=synth.FMT_NVFP4,
                                       down_fmt=synth.FMT_FP8, I_shared=512,
                                       shared_fmt=synth.FMT_FP8,
                                       shared_down_fmt=synth.FMT_NVFP4, zipf_s=1.1),
    "decode_t16_nvfp4_zipf": synth.scaled(W["decode_t8_nvfp4_zipf"], name="decode_t16_nvfp4_zipf",
                                          T=16, weight_sets=1),
    "decode_t12_mxfp4_zipf": synth.scaled(W["decode_t8_mxfp4_zipf"], name="decode_t12_mxfp4_zipf",
                                          T=12, weight_sets=1),
    # every group (and the shared expert) in two chunks of 16 rows
    "nvfp4_t32_full_groups": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_t32_full_groups", T=32,
                                          H=2048, E=4, I=512, top_k=4, I_shared=512,
                                          shared_fmt=synth.FMT_NVFP4),
    "mxfp4_t24_k4096": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_t24_k4096", T=24, H=4096,
                                    E=10, I=512, top_k=2, fmt=synth.FMT_MXFP4, I_shared=1024,
                                    shared_fmt=synth.FMT_FP8, zipf_s=1.1),
    # 500 pair slots (two derivation rounds), groups of ~17 rows
    "nvfp4_t25_k20": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_t25_k20", T=25, H=2048, E=30,
                                  I=512, top_k=20, I_shared=512, shared_fmt=synth.FMT_FP8,
                                  down_fmt=synth.FMT_FP8),
    "decode_t32_nvfp4_zipf": synth.scaled(W["decode_t32_nvfp4_zipf"], name="decode_t32_nvfp4_zipf",
                                          weight_sets=1),
}


@pytest.mark.parametrize("name", list(DECODE_ROWS))
def test_layer_decode_rows(name):
    w = DECODE_ROWS[name]
    say(f"[gpu] layer {name}: T={w.T} H={w.H} E={w.E} I={w.I} k={w.top_k} fmt={w.fmt}")
    tokens = None if w.T <= 16 or w.E <= 64 else [0, 5, 13, 22, 31]
    r = check_layer_against_oracle(layer_for(w), synth.make_x(w), tokens=tokens, what=name)
    counts = np.bincount(r["ids"].reshape(-1), minlength=w.E)
    say(f"[gpu] layer {name}: rel={r['rel']:.2e} worst={r['worst']:.2e} max group={counts.max()}")
    if w.top_k == w.E:
        assert counts.max() == w.T


# The 9-64 row band (speculative-verify and batched-decode sizes): sliced
# router, block top-k, expert GEMV in 16-row passes (groups above 16 rows
# under the Zipf router), shared expert over up to 4 passes.
BAND = {
    "nvfp4_t24": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_t24", T=24, H=352, E=24, I=160,
                              top_k=3, I_shared=96, shared_fmt=synth.FMT_FP8, zipf_s=1.1),
    "mxfp4_t40": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_t40", T=40, H=512, E=16, I=256,
                              top_k=4, fmt=synth.FMT_MXFP4, I_shared=128,
                              shared_fmt=synth.FMT_MXFP4, zipf_s=1.1),
    "fp8_t64": synth.scaled(W["tiny_nvfp4_t4"], name="fp8_t64", T=64, H=336, E=8, I=144,
                            top_k=2, fmt=synth.FMT_FP8, I_shared=272, shared_fmt=synth.FMT_FP8,
                            zipf_s=1.1),
    "nvfp4_t64_decode_shape": synth.scaled(W["decode_t8_nvfp4_zipf"], name="nvfp4_t64_band",
                                           T=64, weight_sets=1),
}


@pytest.mark.parametrize("name", list(BAND))
def test_layer_row_band(name):
    w = BAND[name]
    say(f"[gpu] layer {name}: T={w.T} H={w.H} E={w.E} I={w.I} k={w.top_k} fmt={w.fmt}")
    tokens = None if w.H * w.E <= 512 * 64 else [0, 13, 31, 47, 63]
    r = check_layer_against_oracle(layer_for(w), synth.make_x(w), tokens=tokens, what=name)
    counts = np.bincount(r["ids"].reshape(-1), minlength=w.E)
    say(f"[gpu] layer {name}: rel={r['rel']:.2e} worst={r['worst']:.2e} max group={counts.max()}")
    if w.E <= 24:
        assert counts.max() > 16                 # a group takes more than one 16-row pass


# Per-projection formats (the pages serve layers whose projections mix FP8 and
# FP4): the down projections in another format than gate/up, routed and shared.
MIXED = {
    "nvfp4_gu_fp8_down": synth.scaled(W["tiny_nvfp4_t4"], name="mixed_nv_fp8", T=100, H=352,
                                      E=12, I=160, top_k=3, fmt=synth.FMT_NVFP4,
                                      down_fmt=synth.FMT_FP8, I_shared=96,
                                      shared_fmt=synth.FMT_FP8,
                                      shared_down_fmt=synth.FMT_NVFP4, zipf_s=1.1),
    "mxfp4_gu_nvfp4_down": synth.scaled(W["tiny_nvfp4_t4"], name="mixed_mx_nv", T=100, H=512,
                                        E=10, I=256, top_k=2, fmt=synth.FMT_MXFP4,
                                        down_fmt=synth.FMT_NVFP4, I_shared=128,
                                        shared_fmt=synth.FMT_MXFP4,
                                        shared_down_fmt=synth.FMT_FP8),
}


# Every FP4 projection with K a multiple of 64, routed and shared, so that the
# LDS-DMA grouped GEMM runs all of them (MXFP4 both projections, NVFP4 down)
# at T > 64, the shared expert over its untiled rows included; Zipf groups
# leave single-row and empty experts beside multi-tile ones.
DMA = {
    "mxfp4_all": synth.scaled(W["tiny_nvfp4_t4"], name="dma_mxfp4_all", T=150, H=512, E=10,
                              I=192, top_k=3, fmt=synth.FMT_MXFP4, I_shared=128,
                              shared_fmt=synth.FMT_MXFP4, zipf_s=1.1),
    "nvfp4_all": synth.scaled(W["tiny_nvfp4_t4"], name="dma_nvfp4_all", T=150, H=384, E=10,
                              I=320, top_k=2, fmt=synth.FMT_NVFP4, I_shared=192,
                              shared_fmt=synth.FMT_NVFP4, zipf_s=1.1),
}


@pytest.mark.parametrize("name", list(DMA))
def test_layer_dma_gemm(name):
    w = DMA[name]
    say(f"[gpu] LDS-DMA GEMM layer {name}: T={w.T} H={w.H} I={w.I} shared I={w.I_shared} "
        f"fmt={w.fmt}/{w.shared_fmt}")
    check_layer_against_oracle(layer_for(w), synth.make_x(w), what=name)


# MXFP8 experts (E4M3 codes, E8M0 per 32): routed with ragged and with
# 128-aligned K, and as the shared expert beside NVFP4 routed experts.
MXFP8 = {
    "mxfp8_ragged": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp8_ragged", T=150, H=352, E=12,
                                 I=160, top_k=3, fmt=synth.FMT_MXFP8, I_shared=96,
                                 shared_fmt=synth.FMT_MXFP8, zipf_s=1.1),
    "mxfp8_aligned": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp8_aligned", T=150, H=512, E=10,
                                  I=256, top_k=2, fmt=synth.FMT_MXFP8, I_shared=128,
                                  shared_fmt=synth.FMT_FP8),
    "nvfp4_mxfp8_shared": synth.scaled(W["tiny_nvfp4_t4"], name="nvfp4_mxfp8_shared", T=150,
                                       H=512, E=10, I=256, top_k=2, fmt=synth.FMT_NVFP4,
                                       I_shared=128, shared_fmt=synth.FMT_MXFP8),
}


@pytest.mark.parametrize("name", list(MXFP8))
@pytest.mark.parametrize("T", [1, 5, 40, 150])
def test_layer_mxfp8(name, T):
    """Fused decode (T <= 8), expert GEMV (T = 40) and grouped GEMM (T = 150)."""
    w = MXFP8[name]
    say(f"[gpu] MXFP8 layer {name} T={T}")
    check_layer_against_oracle(layer_for(w), synth.make_x(w)[:T], what=f"{name} T={T}")


@pytest.mark.parametrize("name", list(MIXED))
@pytest.mark.parametrize("T", [1, 5, 12, 40, 100])
def test_layer_mixed_formats(name, T):
    """Fused decode (T <= 8), expert GEMV (T <= 64) and grouped GEMM (T = 100)."""
    w = MIXED[name]
    L = layer_for(w)
    x_bits = synth.make_x(w)[:T]
    say(f"[gpu] mixed formats {name} T={T}: gate/up {w.fmt}, down {w.down_fmt}, "
        f"shared {w.shared_fmt}/{w.shared_down_fmt}")
    check_layer_against_oracle(L, x_bits, what=f"{name} T={T}")


@pytest.mark.parametrize("name", list(MID))
def test_layer_grouped_gemm(name):
    w = MID[name]
    say(f"[gpu] layer {name}: T={w.T} H={w.H} E={w.E} I={w.I} k={w.top_k} fmt={w.fmt}")
    r = check_layer_against_oracle(layer_for(w), synth.make_x(w), what=name)
    counts = np.bincount(r["ids"].reshape(-1), minlength=w.E)
    say(f"[gpu] layer {name}: rel={r['rel']:.2e} worst={r['worst']:.2e} groups={counts.tolist()}")
    assert counts.max() > 128                # at least one group spans two row tiles


# Group sizes around the 128-row tile: empty, 1, one short of a tile, exactly
# one, one over, exactly two, and a ragged multi-tile group.
EDGE_COUNTS = [0, 1, 127, 128, 129, 0, 256, 300]


@pytest.mark.parametrize("fmt,H,I", [(synth.FMT_NVFP4, 352, 160), (synth.FMT_MXFP4, 416, 224),
                                     (synth.FMT_FP8, 336, 144),
                                     # K % 64 == 0: the LDS-DMA kernel (128 x 256
                                     # tiles, 1 x 4 wavefront grid for both FP4
                                     # formats), ragged column tails
                                     (synth.FMT_MXFP4, 384, 224), (synth.FMT_MXFP4, 448, 320),
                                     (synth.FMT_NVFP4, 480, 192), (synth.FMT_NVFP4, 448, 224)])
def test_grouped_gemm_tile_edges(fmt, H, I):
    """moe_expert_gemm on a hand-made grouping (k = 1, tokens shuffled)."""
    E = len(EDGE_COUNTS)
    T = sum(EDGE_COUNTS)
    w = synth.scaled(W["tiny_nvfp4_t4"], name=f"edges_{fmt}", T=T, H=H, E=E, I=I, top_k=1, fmt=fmt)
    say(f"[gpu] grouped GEMM tile edges fmt={fmt} T={T} H={H} I={I} counts={EDGE_COUNTS}")
    L = layer_for(w)
    rng = np.random.default_rng(5)
    ids = rng.permutation(np.repeat(np.arange(E), EDGE_COUNTS)).astype(np.int32).reshape(T, 1)
    G = O.permute(ids, E)
    assert np.array_equal(G.counts, EDGE_COUNTS)
    x_bits = synth.make_x(w)
    x64 = O.bf16_value(x_bits)
    dl = device_layer(L)
    ws = dl.workspace(T)
    offs = torch.from_numpy(G.offsets).cuda()
    p2 = torch.from_numpy(G.perm_to_pair).cuda()
    h = torch.empty((T, I), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_gemm(moe.MOE_OP_GATE_UP_SWIGLU, dl.desc, 0, offs, p2, None, T,
                        bf16_tensor(x_bits), h, ws)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.moe_expert_gemm(moe.MOE_OP_DOWN, dl.desc, 0, offs, p2, None, T, h, y, ws)
    torch.cuda.synchronize()
    got_h = O.bf16_value(bf16_bits(h))
    got_y = y.cpu().numpy()
    ref_h = np.zeros((T, I))
    ref_y = np.zeros((T, H))
    for e in range(E):
        rows = np.arange(G.offsets[e], G.offsets[e + 1])
        if rows.size == 0:
            continue
        toks = G.perm_to_pair[rows]        # k = 1: pair index = token
        ref_h[rows] = O.ffn_gate_up(x64[toks], F.dequant(L.gate, e), F.dequant(L.up, e))
        # down from the GPU's own h, so one bf16 rounding step of h does not
        # propagate into y
        ref_y[rows] = O.ffn_down(got_h[rows], F.dequant(L.down, e))
    assert_close(got_h, ref_h, f"edges {fmt} h")
    assert_close(got_y, ref_y, f"edges {fmt} y")


@pytest.mark.parametrize("name", ["nvfp4_ragged", "fp8_mid"])
def test_layer_is_deterministic(name):
    w = SMALL.get(name) or MID[name]
    dl = device_layer(layer_for(w))
    from gpu_util import run_layer
    x = synth.make_x(w)
    a = run_layer(dl, x)
    b = run_layer(dl, x)
    for u, v in zip(a, b):
        assert np.array_equal(u, v, equal_nan=True)


@pytest.mark.parametrize("T,E,k", [(37, 64, 6), (9, 64, 6), (11, 1000, 12), (40, 300, 32)])
def test_route_topk_given_logits_exact(T, E, k):
    """Given logits: per-token block selection (T <= 16) and per-wavefront
    selection (larger T), on ties, duplicates, NaN and infinities."""
    rng = np.random.default_rng(11 + T)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, [5, 9, 40]] = 9.0
    logits[1, :] = 0.5
    logits[2, [1, 2]] = np.nan
    logits[3, 17] = np.inf
    logits[4, :] = np.round(logits[4, :], 1)        # many exact duplicates
    logits[5, ::2] = np.nan                          # half NaN
    logits[6, :] = -np.inf
    logits[6, 3] = -0.0
    logits[6, 4] = 0.0
    logits[7, :] = np.float32(1.0) + np.arange(E, dtype=np.float32) * np.float32(2**-23)
    w_ = synth.scaled(W["tiny_nvfp4_t4"], name="route", E=E, top_k=k)
    dl = device_layer(layer_for(w_))
    lg = torch.from_numpy(logits).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route_topk(dl.desc, None, lg, T, ids, wt, dl.workspace(T))
    torch.cuda.synchronize()
    ref_ids, ref_w = O.route_from_logits(logits, k, True)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ok = np.all(np.isfinite(ref_w), axis=1)
    assert_close(wt.cpu().numpy()[ok], ref_w[ok], "given-logit weights")


def _tie_router(H, E, seed=3):
    """Router weights with exact ties (duplicated columns) and 1-ulp near
    ties, biased so that the tied experts sit at the top-k boundary."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((H, E)) * 0.05).astype(np.float32)
    w[:, 10] = w[:, 3]                          # exact tie with expert 3
    w[:, 20] = w[:, 3]
    w[7, 20] = np.nextafter(w[7, 3], np.float32(1))   # near tie
    w[:, 33] = w[:, 12]
    b = np.zeros(E, dtype=np.float32)
    b[[3, 10, 20, 12, 33]] = [2.0, 2.0, 2.0, 1.5, 1.5]
    return w, b


def _special_rows(x_bits):
    x = x_bits.copy()
    x[1, 5] = 0x7F80            # +inf
    x[2, 9] = 0x7FC0            # NaN
    x[3, :] = 0                 # all zero: logits = bias, exact ties
    x[4, :] = 0x7F7F            # bf16 max: fp32 sums overflow
    x[5, 17] = 0xFF80           # -inf
    return x


@pytest.mark.parametrize("T", [12, 40])
def test_route_certified_ties_and_specials(T):
    """moe_route_topk from activations (float64 router for T <= 16, matrix-core
    router above) on ties, near ties and non-finite / overflowing rows."""
    H, E, k = 352, 64, 6
    w_ = synth.scaled(W["tiny_nvfp4_t4"], name="route_ties", T=T, H=H, E=E, top_k=k)
    import dataclasses
    wr, b = _tie_router(H, E)
    L = dataclasses.replace(layer_for(w_), router_w=wr, router_bias=b)
    x_bits = _special_rows(synth.make_x(w_))
    say(f"[gpu] route ties/specials T={T}")
    dl = device_layer(L)
    x = bf16_tensor(x_bits)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route_topk(dl.desc, x, lg, T, ids, wt, dl.workspace(T))
    torch.cuda.synchronize()
    ref = O.route(x_bits, wr, b, k, True)
    got = ids.cpu().numpy()
    bad = np.nonzero(np.any(got != ref.ids, axis=1))[0]
    assert bad.size == 0, f"tokens {bad}: got {got[bad[:3]]} want {ref.ids[bad[:3]]}"
    assert_close(wt.cpu().numpy(), ref.weights, "tie routing weights")
    say(f"[gpu] route ties T={T}: oracle recomputed {int(ref.recomputed.sum())} of {T} tokens")


def test_decode_route_ties_and_specials():
    """The fused decode path (T = 8) on the same rows: expert ids exact."""
    H, E, k, T = 352, 64, 6, 8
    w_ = synth.scaled(W["tiny_nvfp4_t4"], name="route_ties", T=T, H=H, E=E, top_k=k)
    import dataclasses
    wr, b = _tie_router(H, E)
    L = dataclasses.replace(layer_for(w_), router_w=wr, router_bias=b)
    x_bits = _special_rows(synth.make_x(w_))
    say("[gpu] decode route ties/specials T=8")
    dl = device_layer(L)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    moe.moe_layer_forward(dl.desc, bf16_tensor(x_bits), T, out, dl.workspace(T), dbg_ids=ids)
    torch.cuda.synchronize()
    ref = O.route(x_bits, wr, b, k, True)
    assert np.array_equal(ids.cpu().numpy(), ref.ids)


@pytest.mark.parametrize("T,k,E,skew", [(1, 10, 512, 0), (8, 10, 512, 1), (300, 7, 96, 1),
                                        (8192, 10, 512, 1), (1500, 1, 3, 0)])
def test_permute_bit_exact(T, k, E, skew):
    say(f"[gpu] permute T={T} k={k} E={E} skew={skew}")
    rng = np.random.default_rng(T * 31 + E)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    ids = ids.astype(np.int32)
    ref = O.permute(ids, E)
    d = torch.from_numpy(ids).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    p2 = torch.empty(T * k, dtype=torch.int32, device="cuda")
    q2 = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_permute_workspace_size(T, k, E), dtype=torch.uint8, device="cuda")
    act = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    moe.moe_permute(d, T, k, E, counts, offsets, p2, q2, act, ws)
    torch.cuda.synchronize()
    a = act.cpu().numpy()
    nz = np.nonzero(ref.counts)[0]
    assert a[0] == nz.size and np.array_equal(a[1:1 + nz.size], nz)
    assert np.array_equal(counts.cpu().numpy(), ref.counts)
    assert np.array_equal(offsets.cpu().numpy(), ref.offsets)
    assert np.array_equal(p2.cpu().numpy(), ref.perm_to_pair)
    assert np.array_equal(q2.cpu().numpy(), ref.pair_to_perm)


@pytest.mark.parametrize("name", ["nvfp4_ragged", "mxfp4_ragged", "fp8_ragged", "nvfp4_aligned",
                                  "mxfp4_aligned"])
def test_expert_gemm_and_combine_units(name):
    """Each unit entry point alone, fed the oracle's own routing."""
    w = SMALL[name]
    L = layer_for(w)
    x_bits = synth.make_x(w)
    ref = O.layer_forward(L, x_bits)
    G = ref.grouping
    dl = device_layer(L)
    T, k, H, I = w.T, w.top_k, w.H, w.I
    P = T * k
    x = bf16_tensor(x_bits)
    offs = torch.from_numpy(G.offsets).cuda()
    p2 = torch.from_numpy(G.perm_to_pair).cuda()
    q2 = torch.from_numpy(G.pair_to_perm).cuda()
    ws = dl.workspace(T)
    h = torch.empty((P, I), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_gemm(moe.MOE_OP_GATE_UP_SWIGLU, dl.desc, 0, offs, p2, None, T, x, h, ws)
    torch.cuda.synchronize()
    pairs = G.perm_to_pair
    ref_h = ref.h.reshape(P, I)[pairs]           # oracle h in permuted order
    got_h = O.bf16_value(bf16_bits(h))
    assert_close(got_h, ref_h, name + " h")
    # down on the oracle's h
    hin = bf16_tensor(O.bf16_bits(ref_h))
    y = torch.empty((P, H), dtype=torch.float32, device="cuda")
    nz = np.nonzero(G.counts)[0]
    act = torch.from_numpy(np.concatenate([[nz.size], nz]).astype(np.int32)).cuda()
    moe.moe_expert_gemm(moe.MOE_OP_DOWN, dl.desc, 0, offs, p2, act, T, hin, y, ws)
    torch.cuda.synchronize()
    yp = np.zeros((P, H))
    for e in np.unique(ref.routing.ids):
        rows = np.arange(G.offsets[e], G.offsets[e + 1])
        yp[rows] = O.ffn_down(ref_h[rows], F.dequant(L.down, int(e)))
    assert_close(y.cpu().numpy(), yp, name + " y")
    # shared expert
    ys = None
    if L.has_shared:
        hs = torch.empty((T, w.I_shared), dtype=torch.bfloat16, device="cuda")
        moe.moe_expert_gemm(moe.MOE_OP_GATE_UP_SWIGLU, dl.desc, 1, None, None, None, T, x, hs, ws)
        ys = torch.empty((T, H), dtype=torch.float32, device="cuda")
        moe.moe_expert_gemm(moe.MOE_OP_DOWN, dl.desc, 1, None, None, None, T,
                            bf16_tensor(O.bf16_bits(ref.h_shared)), ys, ws)
        torch.cuda.synchronize()
        assert_close(O.bf16_value(bf16_bits(hs)), ref.h_shared, name + " shared h")
        assert_close(ys.cpu().numpy(), ref.y_shared, name + " shared y")
    # combine on the oracle's partials
    yperm = torch.from_numpy(ref.y.reshape(P, H)[pairs].astype(np.float32)).cuda()
    wt = torch.from_numpy(ref.routing.weights.astype(np.float32)).cuda()
    ysh = torch.from_numpy(ref.y_shared.astype(np.float32)).cuda() if L.has_shared else None
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(yperm, wt, q2, ysh, T, k, H, out)
    torch.cuda.synchronize()
    assert_close(O.bf16_value(bf16_bits(out)), ref.out, name + " combine")


@pytest.mark.parametrize("name", ["nvfp4_ragged", "mxfp4_ragged", "fp8_ragged", "nvfp4_t3_k1",
                                  "decode_t1_nvfp4", "decode_t8_mxfp4_zipf"])
def test_decode_gate_up_unit(name):
    """moe_decode_gate_up (the decode lowering's gate/up launch, timed by the
    bench) on the oracle's routing: every routed h row and the shared h."""
    w = SMALL.get(name) or W[name]
    L = layer_for(w)
    x_bits = synth.make_x(w)[:min(w.T, 8)]
    T, k, I = x_bits.shape[0], w.top_k, w.I
    say(f"[gpu] decode gate/up unit {name}: T={T} H={w.H} I={I} k={k} fmt={w.fmt}")
    ref = O.layer_forward(L, x_bits)
    dl = device_layer(L)
    ids = torch.from_numpy(ref.routing.ids).cuda()
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device="cuda")
    hs = torch.empty((T, w.I_shared), dtype=torch.bfloat16, device="cuda") if L.has_shared else None
    moe.moe_decode_gate_up(dl.desc, bf16_tensor(x_bits), T, ids, h, hs)
    torch.cuda.synchronize()
    assert_close(O.bf16_value(bf16_bits(h)), ref.h.reshape(T * k, I), name + " decode h")
    if L.has_shared:
        assert_close(O.bf16_value(bf16_bits(hs)), ref.h_shared, name + " decode shared h")


@pytest.mark.parametrize("name", ["nvfp4_t32_full_groups", "mxfp4_t24_k4096"])
def test_decode_gate_up_unit_rows(name):
    """moe_decode_gate_up at 24 and 32 rows on aligned shapes (groups taken
    in chunks of 16 rows), and MOE_ERR_UNSUPPORTED at 12 rows of a shape whose
    layer runs the expert GEMV instead."""
    w = DECODE_ROWS[name]
    L = layer_for(w)
    x_bits = synth.make_x(w)
    T, k, I = w.T, w.top_k, w.I
    say(f"[gpu] decode gate/up unit {name}: T={T} H={w.H} I={I} k={k} fmt={w.fmt}")
    ref = O.layer_forward(L, x_bits)
    dl = device_layer(L)
    ids = torch.from_numpy(ref.routing.ids).cuda()
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device="cuda")
    hs = torch.empty((T, w.I_shared), dtype=torch.bfloat16, device="cuda") if L.has_shared else None
    moe.moe_decode_gate_up(dl.desc, bf16_tensor(x_bits), T, ids, h, hs)
    torch.cuda.synchronize()
    assert_close(O.bf16_value(bf16_bits(h)), ref.h.reshape(T * k, I), name + " decode h")
    if L.has_shared:
        assert_close(O.bf16_value(bf16_bits(hs)), ref.h_shared, name + " decode shared h")
    ws_ = SMALL["nvfp4_t12"]
    L12 = layer_for(ws_)
    dl12 = device_layer(L12)
    x12 = bf16_tensor(synth.make_x(ws_))
    ids12 = torch.zeros((ws_.T, ws_.top_k), dtype=torch.int32, device="cuda")
    h12 = torch.empty((ws_.T * ws_.top_k, ws_.I), dtype=torch.bfloat16, device="cuda")
    hs12 = torch.empty((ws_.T, ws_.I_shared), dtype=torch.bfloat16, device="cuda")
    st = moe.moe_decode_gate_up(dl12.desc, x12, ws_.T, ids12, h12, hs12, check=False)
    assert st == moe.MOE_ERR_UNSUPPORTED


def test_workspace_reuse_across_batch_sizes():
    """One zero-filled workspace, calls with T = 8, 1, 5, 8 in a row: the fused
    decode kernels leave their counters zero, so every call stays exact."""
    from gpu_util import run_layer  # noqa: F401
    w = SMALL["mxfp4_ragged"]
    L = layer_for(w)
    dl = device_layer(L)
    ws = dl.workspace(8)
    x_all = synth.make_x(synth.scaled(w, T=8))
    for T in (8, 1, 5, 8, 3):
        x_bits = x_all[:T]
        x = bf16_tensor(x_bits)
        out = torch.empty((T, w.H), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
        moe.moe_layer_forward(dl.desc, x, T, out, ws, dbg_ids=ids)
        torch.cuda.synchronize()
        ref = O.layer_forward(L, x_bits)
        assert np.array_equal(ids.cpu().numpy(), ref.routing.ids), T
        assert_close(O.bf16_value(bf16_bits(out)), ref.out, f"reuse T={T}")


def _degenerate_layer(fmt, H=352, I=160):
    """A small layer whose routed experts 0..4 (all tokens route to them: a
    +20 router bias, k = 5) carry degenerate weights: a NaN block scale in
    one down-projection row, a NaN element of an FP8 code, subnormal and zero
    scales, maximum-magnitude codes, an all-zero expert, a zero tensor scale,
    and a NaN block scale in the shared expert's down projection."""
    import dataclasses
    w = synth.scaled(W["tiny_nvfp4_t4"], name=f"degenerate_{fmt}_{H}_{I}", T=150, H=H, E=8, I=I,
                     top_k=5, fmt=fmt, I_shared=96, shared_fmt=synth.FMT_FP8)
    L = layer_for(w)

    def clone(q):
        return dataclasses.replace(q, codes=q.codes.copy(), scales=q.scales.copy(),
                                   tensor_scale=None if q.tensor_scale is None else q.tensor_scale.copy())
    gate, up, down, sd = clone(L.gate), clone(L.up), clone(L.down), clone(L.sh_down)
    if fmt == synth.FMT_NVFP4:
        down.scales[0, 5, 1] = 0x7F          # E4M3 NaN: column 5 of expert 0's output
        up.codes[1] = 0x77                   # every code +6 ...
        up.scales[1] = 0x7E                  # ... times the largest scale, 448
        gate.scales[2] = 0x01                # smallest subnormal scale, 2^-9
        down.scales[2, :, ::2] = 0x00        # zero scales in half the blocks
        gate.codes[3] = 0
        up.codes[3] = 0                      # an all-zero expert
        gate.tensor_scale[4] = 0.0           # zero tensor scale
    elif fmt == synth.FMT_MXFP4:
        down.scales[0, 7, 0] = 0xFF          # E8M0 NaN
        up.scales[1] = 0                     # 2^-127
        gate.codes[2] = 0x77
        gate.scales[2] = 127 + 8             # 6 * 2^8
        gate.codes[3] = 0
        up.codes[3] = 0
    else:
        down.codes[0, 9, 17] = 0x7F          # E4M3 NaN code
        up.codes[1] = 0x7E                   # 448 everywhere ...
        up.scales[1] = 4.0                   # ... times 4
        gate.codes[2] = 0x01                 # smallest subnormal code
        gate.codes[3] = 0
        up.codes[3] = 0
    sd.scales[0, 0, 0] = np.nan              # shared down: rows 0..127 NaN
    bias = np.zeros(w.E, dtype=np.float32)
    bias[:5] = 20.0
    L2 = dataclasses.replace(L, gate=gate, up=up, down=down, sh_down=sd, router_bias=bias)
    return w, L2


@pytest.mark.parametrize("fmt", [synth.FMT_NVFP4, synth.FMT_MXFP4, synth.FMT_FP8])
@pytest.mark.parametrize("T", [5, 12, 40, 80])
def test_degenerate_weights(fmt, T):
    """NaN, subnormal, zero and extreme checkpoint values through the decode
    (T <= 8), expert-GEMV (T <= 64) and grouped-GEMM paths: same NaN pattern
    as the oracle, the finite outputs within tolerance."""
    w, L = _degenerate_layer(fmt)
    x_bits = synth.make_x(w)[:T]
    say(f"[gpu] degenerate weights fmt={fmt} T={T}")
    r = check_layer_against_oracle(L, x_bits, what=f"degenerate {fmt} T={T}")
    assert np.isnan(r["out"]).any() and np.isfinite(r["out"]).any()


@pytest.mark.parametrize("fmt", [synth.FMT_NVFP4, synth.FMT_MXFP4])
@pytest.mark.parametrize("T", [1, 5])
def test_degenerate_weights_k2048(fmt, T):
    """The degenerate values through the decode's aligned FP4 gate/up tile
    (K = H = 2048)."""
    w, L = _degenerate_layer(fmt, H=2048, I=256)
    x_bits = synth.make_x(w)[:T]
    say(f"[gpu] degenerate weights (K = 2048) fmt={fmt} T={T}")
    r = check_layer_against_oracle(L, x_bits, what=f"degenerate k2048 {fmt} T={T}")
    assert np.isnan(r["out"]).any() and np.isfinite(r["out"]).any()


@pytest.mark.parametrize("fmt", [synth.FMT_NVFP4, synth.FMT_MXFP4])
@pytest.mark.parametrize("T", [5, 12, 80, 150])
def test_degenerate_weights_aligned(fmt, T):
    """The same degenerate values with K a multiple of 128, where the FP4
    block scales are read by whole chunk (fused decode at T = 5, the
    small-group expert GEMV at T = 12) and every FP4 projection of the
    grouped GEMM runs the LDS-DMA kernel (T = 80, 150: groups of one and two
    128-row tiles)."""
    w, L = _degenerate_layer(fmt, H=512, I=256)
    x_bits = synth.make_x(w)[:T]
    say(f"[gpu] degenerate weights (aligned K) fmt={fmt} T={T}")
    r = check_layer_against_oracle(L, x_bits, what=f"degenerate aligned {fmt} T={T}")
    assert np.isnan(r["out"]).any() and np.isfinite(r["out"]).any()
