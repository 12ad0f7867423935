"""GPU parity at the full workload shapes: every output compared with the oracle.

The wide-FP8 prefill layer (T=8192, H=6144, I=2048) is the one exception: its
float64 oracle over all 65,536 routed rows would take many minutes, so it is
checked on routing for every token, on every routed row of a sample of experts
through the expert-GEMM entry point (the hottest, the coldest and evenly
spread ones), and on the complete output of two tokens.
"""
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


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode_t8_fp8_wide", "prefill_t8192_nvfp4_zipf",
                                  "prefill_t8192_mxfp4_zipf"])
def test_layer_full_shape_every_output(name):
    """Routing bit-exact for every token and every output element within the
    float bar: the wide-FP8 decode layer (8 tokens, 57+ experts of 37.8 MB)
    and the two T=8192 prefill layers (every (expert, 128-row tile) of the
    grouped GEMMs, the hot Zipf groups of several thousand rows included)."""
    w = W[name]
    say(f"[gpu] full-shape layer {name}: T={w.T} H={w.H} E={w.E} I={w.I} k={w.top_k} fmt={w.fmt}")
    r = check_layer_against_oracle(layer_for(w), synth.make_x(w), what=name)
    counts = np.bincount(r["ids"].reshape(-1), minlength=w.E)
    say(f"[gpu] {name}: all {w.T} tokens, rel={r['rel']:.2e} worst={r['worst']:.2e} "
        f"active experts={int((counts > 0).sum())} max group={int(counts.max())} "
        f"oracle recomputed={r['recomputed']}")
    if w.T > 64:
        assert counts.max() > 128           # a group spans several 128-row tiles


@pytest.mark.timeout(900)
def test_prefill_fp8_wide_sampled_experts_and_tokens():
    w = W["prefill_t8192_fp8_wide"]
    L = layer_for(w)
    x_bits = synth.make_x(w)
    T, k, H, I, E = w.T, w.top_k, w.H, w.I, w.E
    P = T * k
    say(f"[gpu] prefill_t8192_fp8_wide: T={T} H={H} I={I} E={E} k={k} (FP8 block-128, K=6144 / 2048)")
    dl = device_layer(L)
    ws = dl.workspace(T)
    x = bf16_tensor(x_bits)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    moe.moe_layer_forward(dl.desc, x, T, out, ws, dbg_ids=ids)
    torch.cuda.synchronize()
    R = O.route(x_bits, L.router_w, L.router_bias, k, L.renormalize)
    got_ids = ids.cpu().numpy()
    bad = np.nonzero(np.any(got_ids != R.ids, axis=1))[0]
    assert bad.size == 0, f"routing differs for tokens {bad[:10]}"
    G = O.permute(R.ids, E)
    # the expert GEMMs over all routed rows, grouped as the oracle groups them
    offs = torch.from_numpy(G.offsets).cuda()
    p2 = torch.from_numpy(G.perm_to_pair).cuda()
    h = torch.empty((P, I), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_gemm(moe.MOE_OP_GATE_UP_SWIGLU, dl.desc, 0, offs, p2, None, T, x, h, ws)
    y = torch.empty((P, H), dtype=torch.float32, device="cuda")
    moe.moe_expert_gemm(moe.MOE_OP_DOWN, dl.desc, 0, offs, p2, None, T, h, y, ws)
    torch.cuda.synchronize()
    order = np.argsort(G.counts, kind="stable")
    sample = sorted(set(order[-4:].tolist() + order[:4].tolist() +
                        np.linspace(0, E - 1, 8).astype(int).tolist()))
    x64 = O.bf16_value(x_bits)
    dec = O._Decoded(L, maxsize=3 * len(sample) + 32)
    rows_checked = 0
    for e in sample:
        rows = np.arange(G.offsets[e], G.offsets[e + 1])
        if rows.size == 0:
            continue
        toks = G.perm_to_pair[rows] // k
        got_h = O.bf16_value(bf16_bits(h[rows[0]:rows[-1] + 1]))
        ref_h = O.ffn_gate_up(x64[toks], dec("gate", int(e)), dec("up", int(e)))
        assert_close(got_h, ref_h, f"fp8 wide h expert {e}")
        # down on the GPU's own h (one bf16 rounding of h does not propagate)
        got_y = y[rows[0]:rows[-1] + 1].cpu().numpy()
        ref_y = O.ffn_down(got_h, dec("down", int(e)))
        assert_close(got_y, ref_y, f"fp8 wide y expert {e}")
        rows_checked += rows.size
    say(f"[gpu] fp8 wide: {len(sample)} experts, {rows_checked} routed rows checked")
    toks = [0, T - 1]
    ref = O.layer_forward(L, x_bits, tokens=toks, routing=R, decoded=dec)
    got = O.bf16_value(bf16_bits(out))[toks]
    rel, worst = assert_close(got, ref.out, "fp8 wide layer output")
    say(f"[gpu] fp8 wide: outputs of tokens {toks}: rel={rel:.2e} worst={worst:.2e}")
