"""GPU parity of the opt-in lossy activation modes against the mirrored oracle.

* quantizers: codes and scales bit-exact (rounding ties, saturation, zero,
  subnormal, huge and non-finite rows, ragged 128-blocks);
* grouped GEMM on quantized inputs: the oracle's own quantized inputs fed to
  moe_expert_gemm_q, compared with the oracle's exact contraction of the
  dequantized values;
* whole layer: routing bit-exact, output within the float bar of the oracle
  running the same mode.
"""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import layer as O
from oracle import lossy as Q

from gpu_util import assert_close, device_layer, layer_for, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts too
    pytest.skip("no GPU", allow_module_level=True)

import quantized_moe_expert_02_amd as moe  # noqa: E402
from quantized_moe_expert_02_amd.device import bf16_bits, bf16_tensor  # noqa: E402

W = synth.WORKLOADS
MODE = {"mxfp8": moe.MOE_ACT_MXFP8, "mxfp4": moe.MOE_ACT_MXFP4, "fp8_t128": moe.MOE_ACT_FP8_T128}
ELEM = {"mxfp8": "e4m3", "mxfp4": "e2m1"}


# ------------------------------------------------------------------ helpers
def oracle_quantized(values, mode):
    """The oracle's quantized rows in the library's layout: (codes uint8,
    scales bytes [rows][4*ceil(K/128)]) plus the dequantized float64 values."""
    rows, K = values.shape
    nb = (K + 127) // 128
    if mode == "fp8_t128":
        c, s = Q.t128_quantize(values)
        return c, np.ascontiguousarray(s.astype(np.float32)).view(np.uint8), Q.t128_dequantize(c, s)
    c, s = Q.mx_quantize(values, ELEM[mode])
    sp = np.full((rows, 4 * nb), 127, dtype=np.uint8)
    sp[:, :K // 32] = s
    deq = Q.mx_dequantize(c, s, ELEM[mode])
    if mode == "mxfp4":
        c = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return c, sp, deq


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_quantize(mode, x_bits):
    rows, K = x_bits.shape
    nb = (K + 127) // 128
    codes = torch.zeros((rows, K // 2 if mode == "mxfp4" else K), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, 4 * nb), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_act(MODE[mode], bf16_tensor(x_bits), rows, K, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def special_rows(K, seed):
    """bf16 rows covering the quantizers' edge cases."""
    rng = np.random.default_rng(seed)
    n = 24
    v = (rng.standard_normal((n, K)) * np.exp2(rng.integers(-40, 40, (n, 1)))).astype(np.float32)
    v[0] = 0.0                                                    # all-zero row
    v[1] = np.float32(2.0 ** -133) * rng.integers(-3, 4, K)       # bf16 subnormals
    v[2] = (rng.standard_normal(K) * 1e-39).astype(np.float32)    # subnormal / normal mix
    v[3] = (rng.uniform(-1, 1, K) * 3.0e38).astype(np.float32)    # near the top of the range
    v[4, 5] = np.nan
    v[5, min(40, K - 1)] = np.inf
    v[6, 0] = -np.inf
    # rounding ties: E4M3 grid midpoints under scale 2^-8 (block amax 1.0)
    m8 = F.e4m3_value(np.arange(0x7F))
    mid8 = ((m8[:-1] + m8[1:]) / 2) / 256.0
    v[7] = np.resize(np.concatenate([[1.0], mid8, -mid8]), K)
    # E2M1 midpoints under scale 2^-2 (block amax 1.5)
    mid4 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) / 4.0
    v[8] = np.resize(np.concatenate([[1.5], mid4, -mid4]), K)
    v[9] = -0.0
    v[10] = np.resize([1.9, 0.3, -0.7], K)                        # saturating blocks
    bits = synth.bf16_bits_from_f32(v)
    return bits


# ------------------------------------------------------------------ quantizers
@pytest.mark.parametrize("mode", list(MODE))
@pytest.mark.parametrize("K", [352, 256, 32])
def test_quantize_bit_exact(mode, K):
    x = special_rows(K, seed=K)
    say(f"[lossy] quantize mode={mode} K={K}")
    got_c, got_s = gpu_quantize(mode, x)
    ref_c, ref_s, _ = oracle_quantized(O.bf16_value(x), mode)
    assert np.array_equal(got_c, ref_c), np.argwhere(got_c != ref_c)[:8]
    if mode == "fp8_t128":
        nb = (K + 127) // 128
        g = got_s[:, :4 * nb].view(np.uint32)
        r = ref_s.view(np.uint32)
        gn, rn = np.isnan(g.view(np.float32)), np.isnan(r.view(np.float32))
        assert np.array_equal(gn, rn)
        assert np.array_equal(g[~gn], r[~rn])
    else:
        assert np.array_equal(got_s, ref_s), np.argwhere(got_s != ref_s)[:8]


def test_quantize_rejects_bad_arguments():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 4), dtype=torch.uint8, device="cuda")
    assert moe.moe_quantize_act(7, x, 4, 64, c, s, check=False) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_quantize_act(1, x, 4, 48, c, s, check=False) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_quantize_act(1, x, 0, 64, c, s, check=False) == moe.MOE_OK


# ------------------------------------------------------------------ GEMM units
UNIT = {
    "mxfp4_unit": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_unit", T=150, H=416, E=6, I=224,
                               top_k=3, fmt=synth.FMT_MXFP4, I_shared=96,
                               shared_fmt=synth.FMT_MXFP4, zipf_s=1.1),
    "fp8_unit": synth.scaled(W["tiny_nvfp4_t4"], name="fp8_unit", T=140, H=352, E=5, I=288,
                             top_k=2, fmt=synth.FMT_FP8, I_shared=160, shared_fmt=synth.FMT_FP8),
}


@pytest.mark.parametrize("name,mode", [("mxfp4_unit", "mxfp8"), ("mxfp4_unit", "mxfp4"),
                                       ("fp8_unit", "fp8_t128")])
def test_expert_gemm_q_units(name, mode):
    """moe_expert_gemm_q fed the oracle's quantized inputs and routing."""
    w = UNIT[name]
    L = layer_for(w)
    x_bits = synth.make_x(w)
    R = O.route(x_bits, L.router_w, L.router_bias, w.top_k, w.renormalize)
    G = O.permute(R.ids, L.E)
    dl = device_layer(L)
    T, k, H, I = w.T, w.top_k, w.H, w.I
    P = T * k
    say(f"[lossy] gemm units {name} mode={mode}")
    xc, xs, xdeq = oracle_quantized(O.bf16_value(x_bits), mode)
    offs, p2 = dev(G.offsets), dev(G.perm_to_pair)
    ws = dl.workspace(T)
    h = torch.empty((P, I), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_gemm_q(MODE[mode], moe.MOE_OP_GATE_UP_SWIGLU, dl.desc, 0, offs, p2, None, T,
                          dev(xc), dev(xs), h, ws)
    torch.cuda.synchronize()
    tok = G.perm_to_pair // k
    ref_h = np.zeros((P, I))
    for e in np.nonzero(G.counts)[0]:
        rows = np.arange(G.offsets[e], G.offsets[e + 1])
        ref_h[rows] = O.ffn_gate_up(xdeq[tok[rows]], F.dequant(L.gate, int(e)),
                                    F.dequant(L.up, int(e)))
    assert_close(O.bf16_value(bf16_bits(h)), ref_h, f"{name} {mode} h")
    # down on the oracle's quantized h
    hc, hs_, hdeq = oracle_quantized(ref_h, mode)
    y = torch.empty((P, H), dtype=torch.float32, device="cuda")
    moe.moe_expert_gemm_q(MODE[mode], moe.MOE_OP_DOWN, dl.desc, 0, offs, p2, None, T, dev(hc),
                          dev(hs_), y, ws)
    torch.cuda.synchronize()
    ref_y = np.zeros((P, H))
    for e in np.nonzero(G.counts)[0]:
        rows = np.arange(G.offsets[e], G.offsets[e + 1])
        ref_y[rows] = hdeq[rows] @ F.dequant(L.down, int(e)).T
    assert_close(y.cpu().numpy(), ref_y, f"{name} {mode} y")
    # shared expert (same format family as the routed one here)
    hsh = torch.empty((T, w.I_shared), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_gemm_q(MODE[mode], moe.MOE_OP_GATE_UP_SWIGLU, dl.desc, 1, None, None, None, T,
                          dev(xc), dev(xs), hsh, ws)
    torch.cuda.synchronize()
    ref_hs = O.ffn_gate_up(xdeq, F.dequant(L.sh_gate, 0), F.dequant(L.sh_up, 0))
    assert_close(O.bf16_value(bf16_bits(hsh)), ref_hs, f"{name} {mode} shared h")


def test_expert_gemm_q_rejects_other_formats():
    w = synth.scaled(W["tiny_nvfp4_t4"], name="nv_q", T=20)
    dl = device_layer(layer_for(w))
    c = torch.zeros((20, 256), dtype=torch.uint8, device="cuda")
    s = torch.zeros((20, 8), dtype=torch.uint8, device="cuda")
    out = torch.zeros((20, 128), dtype=torch.bfloat16, device="cuda")
    st = moe.moe_expert_gemm_q(moe.MOE_ACT_MXFP8, moe.MOE_OP_GATE_UP_SWIGLU, dl.desc, 0,
                               torch.zeros(9, dtype=torch.int32, device="cuda"),
                               torch.zeros(40, dtype=torch.int32, device="cuda"), None, 20, c, s,
                               out, dl.workspace(20), check=False)
    assert st == moe.MOE_ERR_UNSUPPORTED


# ------------------------------------------------------------------ whole layer
LAYERS = {
    # K tails (416 = 3 * 128 + 32, 224), column tails, MX shared expert
    "mxfp4_mid": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_mid_q", T=200, H=416, E=5, I=224,
                              top_k=2, fmt=synth.FMT_MXFP4, I_shared=64,
                              shared_fmt=synth.FMT_MXFP4, zipf_s=1.1),
    # K multiples of 128, FP8 shared expert (kept exact by the MX modes)
    "mxfp4_aligned": synth.scaled(W["tiny_nvfp4_t4"], name="mxfp4_aligned_q", T=300, H=1024,
                                  E=8, I=384, top_k=3, fmt=synth.FMT_MXFP4, I_shared=256,
                                  shared_fmt=synth.FMT_FP8),
    "fp8_mid": synth.scaled(W["tiny_nvfp4_t4"], name="fp8_mid_q", T=260, H=352, E=4, I=160,
                            top_k=2, fmt=synth.FMT_FP8, I_shared=288, shared_fmt=synth.FMT_FP8),
    # K multiples of 128: the LDS-DMA kernels (whole steps only)
    "fp8_aligned": synth.scaled(W["tiny_nvfp4_t4"], name="fp8_aligned_q", T=230, H=512, E=6,
                                I=256, top_k=2, fmt=synth.FMT_FP8, I_shared=384,
                                shared_fmt=synth.FMT_FP8),
}


def run_layer_ex(dl, x_bits, mode_code):
    L = dl.L
    T = x_bits.shape[0]
    out = torch.empty((T, L.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
    moe.moe_layer_forward_ex(dl.desc, bf16_tensor(x_bits), T, out, dl.workspace(T), mode_code,
                             dbg_ids=ids, dbg_w=wts)
    torch.cuda.synchronize()
    return O.bf16_value(bf16_bits(out)), ids.cpu().numpy(), wts.cpu().numpy()


@pytest.mark.parametrize("name,mode", [("mxfp4_mid", "mxfp8"), ("mxfp4_mid", "mxfp4"),
                                       ("mxfp4_aligned", "mxfp8"), ("mxfp4_aligned", "mxfp4"),
                                       ("fp8_mid", "fp8_t128"), ("fp8_aligned", "fp8_t128")])
def test_layer_lossy_modes(name, mode):
    w = LAYERS[name]
    L = layer_for(w)
    x_bits = synth.make_x(w)
    say(f"[lossy] layer {name} mode={mode} T={w.T}")
    out, ids, wts = run_layer_ex(device_layer(L), x_bits, MODE[mode])
    ref = Q.layer_forward(L, x_bits, mode)
    assert np.array_equal(ids, ref.routing.ids)
    rel, worst = assert_close(out, ref.out, f"{name} {mode} output")
    exact = O.layer_forward(L, x_bits, routing=ref.routing)
    d_mode = np.linalg.norm(ref.out64 - exact.out64) / np.linalg.norm(exact.out64)
    say(f"[lossy] {name} {mode}: rel {rel:.2e} worst {worst:.2e}; mode vs exact chain {d_mode:.2e}")


def test_layer_mode_small_batches_are_exact():
    """T <= 64: the mode does not apply; the result is moe_layer_forward's, bit for bit."""
    w = synth.scaled(LAYERS["mxfp4_mid"], name="mxfp4_small_q", T=12)
    dl = device_layer(layer_for(w))
    x_bits = synth.make_x(w)
    a, _, _ = run_layer_ex(dl, x_bits, moe.MOE_ACT_MXFP8)
    b, _, _ = run_layer_ex(dl, x_bits, moe.MOE_ACT_EXACT)
    assert np.array_equal(a, b)


def test_layer_mode_needs_whole_32_blocks():
    """An FP8 layer whose K is not a multiple of 32 has no 1x128 mode."""
    w = synth.scaled(W["tiny_nvfp4_t4"], name="fp8_k16_q", T=40, H=336, E=4, I=160, top_k=2,
                     fmt=synth.FMT_FP8)
    dl = device_layer(layer_for(w))
    x = bf16_tensor(synth.make_x(w))
    out = torch.empty((40, w.H), dtype=torch.bfloat16, device="cuda")
    st = moe.moe_layer_forward_ex(dl.desc, x, 40, out, dl.workspace(40), moe.MOE_ACT_FP8_T128,
                                  check=False)
    assert st == moe.MOE_ERR_UNSUPPORTED


def test_layer_mode_needs_a_matching_format():
    w = synth.scaled(W["tiny_nvfp4_t4"], name="nv_layer_q", T=40)
    dl = device_layer(layer_for(w))
    x = bf16_tensor(synth.make_x(w))
    out = torch.empty((40, w.H), dtype=torch.bfloat16, device="cuda")
    for m, want in ((moe.MOE_ACT_MXFP8, moe.MOE_ERR_UNSUPPORTED), (9, moe.MOE_ERR_INVALID_ARG)):
        st = moe.moe_layer_forward_ex(dl.desc, x, 40, out, dl.workspace(40), m, check=False)
        assert st == want
