"""GPU edge cases: E8M0 scale codes 0x00 and 0xFF in every lowering, and a
workspace whose bytes hold garbage before the call.

E8M0 (OCP Microscaling Formats v1.0): code 0xFF is NaN and code 0x00 is
2^-127.  The kernels hand the code to the gfx950 scaled converters as the
fp32 bit pattern code << 23; those converters take only the exponent field
of that operand as the scale, so 0x00 scales by 2^-127 and 0xFF gives NaN
(measured on MI355X for every E2M1 code and a range of E4M3 codes).  These
tests pin both ends against the oracle where a +0 or +Inf reading of the
bit pattern would differ:
  * down row 5, K block 0: scale 0xFF over all-positive codes and an
    all-positive input block, so the oracle's NaN differs from +Inf;
  * down row 7, K block 1: scale 0x00 over the largest code, times input
    2^126, so that block alone contributes 96 (E2M1 6) or 32 (E4M3 2), far
    above the tolerance, and a flush to zero would fail.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import layer as O

from gpu_util import assert_close, check_layer_against_oracle, device_layer, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts too
    pytest.skip("no GPU", allow_module_level=True)

import quantized_moe_expert_02_amd as moe  # noqa: E402
from quantized_moe_expert_02_amd.device import bf16_bits, bf16_tensor  # noqa: E402

W = synth.WORKLOADS
BIG = 0x7E80   # bf16 2^126
ONE = 0x3F80   # bf16 1.0


def _e8m0_layer(fmt, I, H=512, T=150):
    """Two routed experts, k = 1, the router biased to expert 0; expert 0's
    down projection carries the two E8M0 edge blocks described above."""
    w = synth.scaled(W["tiny_nvfp4_t4"], name=f"e8m0_{fmt}_{I}", T=T, H=H, E=2, I=I, top_k=1,
                     fmt=fmt)
    L = synth.make_layer(w)
    down = dataclasses.replace(L.down, codes=L.down.codes.copy(), scales=L.down.scales.copy())
    c, s = down.codes[0], down.scales[0]
    if fmt == synth.FMT_MXFP4:            # two codes per byte, K block = 16 bytes
        c[:, 16:32] = 0                   # no row sees K block 1 ...
        c[7, :] = 0
        c[7, 16:32] = 0x77                # ... but row 7: +6 everywhere in it
        c[5, 0:16] = 0x22                 # row 5, K block 0: +1.0 everywhere
    else:                                 # MXFP8: one E4M3 code per byte
        c[:, 32:64] = 0
        c[7, :] = 0
        c[7, 32:64] = 0x40                # +2.0
        c[5, 0:32] = 0x38                 # +1.0
    s[7, 1] = 0x00                        # 2^-127
    s[5, 0] = 0xFF                        # NaN
    bias = np.array([20.0, -20.0], dtype=np.float32)
    return w, dataclasses.replace(L, down=down, router_bias=bias)


def _edge_input(T, I, seed=3):
    rng = np.random.default_rng(seed)
    h = O.bf16_bits(O.round_bf16(rng.standard_normal((T, I))))
    h[:, 0:32] = ONE
    h[:, 32:64] = BIG
    return h


@pytest.mark.parametrize("fmt", [synth.FMT_MXFP4, synth.FMT_MXFP8])
@pytest.mark.parametrize("I", [256, 160])       # whole 128-K chunks / a K tail
@pytest.mark.parametrize("T", [5, 40, 150])     # expert GEMV / GEMV / grouped GEMM
def test_e8m0_edge_codes_down_projection(fmt, I, T):
    w, L = _e8m0_layer(fmt, I)
    say(f"[gpu] E8M0 edges fmt={fmt} K={I} T={T}")
    dl = device_layer(L)
    ws = dl.workspace(T)
    hb = _edge_input(T, I)
    offs = torch.tensor([0, T, T], dtype=torch.int32, device="cuda")
    p2 = torch.arange(T, dtype=torch.int32, device="cuda")
    y = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    moe.moe_expert_gemm(moe.MOE_OP_DOWN, dl.desc, 0, offs, p2, None, T, bf16_tensor(hb), y, ws)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    ref = O.ffn_down(O.bf16_value(hb), F.dequant(L.down, 0))
    assert np.all(np.isnan(ref[:, 5])) and np.all(np.isfinite(np.delete(ref, 5, axis=1)))
    assert np.all(ref[:, 7] == (96.0 if fmt == synth.FMT_MXFP4 else 32.0))
    assert_close(got, ref, f"E8M0 edges {fmt} K={I} T={T}")


@pytest.mark.parametrize("fmt", [synth.FMT_MXFP4, synth.FMT_MXFP8])
@pytest.mark.parametrize("T", [1, 5])
def test_e8m0_nan_scale_in_decode_layer(fmt, T):
    """The fused decode's down-combine on the same expert: output column 5 is
    NaN for every token, as in the oracle; the rest within tolerance."""
    w, L = _e8m0_layer(fmt, 256)
    say(f"[gpu] E8M0 NaN scale through the decode layer fmt={fmt} T={T}")
    r = check_layer_against_oracle(L, synth.make_x(w)[:T], what=f"E8M0 decode {fmt} T={T}")
    assert np.all(np.isnan(r["out"][:, 5]))


@pytest.mark.parametrize("T", [1, 5, 8, 40, 150])
def test_workspace_needs_no_initialisation(T):
    """The layer on a workspace filled with 0xFF bytes (twice in a row) matches
    the oracle: no kernel reads a workspace byte it has not written in the
    same call."""
    w = synth.scaled(W["tiny_nvfp4_t4"], name="ws_garbage", T=150, H=512, E=10, I=256, top_k=3,
                     fmt=synth.FMT_MXFP4, I_shared=128, shared_fmt=synth.FMT_FP8, zipf_s=1.1)
    L = synth.make_layer(w)
    dl = device_layer(L)
    x_bits = synth.make_x(w)[:T]
    ws = torch.full((moe.moe_workspace_size(dl.desc, T),), 0xFF, dtype=torch.uint8, device="cuda")
    ref = O.layer_forward(L, x_bits)
    say(f"[gpu] 0xFF-filled workspace T={T}")
    for rep in range(2):
        out = torch.empty((T, w.H), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
        moe.moe_layer_forward(dl.desc, bf16_tensor(x_bits), T, out, ws, dbg_ids=ids)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ref.routing.ids), (T, rep)
        assert_close(O.bf16_value(bf16_bits(out)), ref.out, f"0xFF workspace T={T} call {rep}")
        ws.fill_(0xFF)
