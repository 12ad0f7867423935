"""Graph capture: moe_layer_forward(_ex) captured into a HIP graph gives the
eager result bit for bit on every replay, with eager work between replays."""
import numpy as np
import pytest

import synth

from gpu_util import device_layer, layer_for, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts too
    pytest.skip("no GPU", allow_module_level=True)

import quantized_moe_expert_02_amd as moe  # noqa: E402
from quantized_moe_expert_02_amd.device import bf16_tensor  # noqa: E402

W = synth.WORKLOADS
LAYER = synth.scaled(W["tiny_nvfp4_t4"], name="graph_layer", T=200, H=512, E=10, I=256, top_k=2,
                     fmt=synth.FMT_MXFP4, I_shared=128, shared_fmt=synth.FMT_FP8, zipf_s=1.1)


@pytest.mark.parametrize("T,mode", [(5, 0), (40, 0), (200, 0), (200, 1)])
def test_graph_replays_match_eager(T, mode):
    dl = device_layer(layer_for(LAYER))
    x = bf16_tensor(synth.make_x(LAYER)[:T])
    ws = dl.workspace(T)
    out = torch.empty((T, LAYER.H), dtype=torch.bfloat16, device="cuda")
    say(f"[gpu] graph capture T={T} mode={mode}")
    moe.moe_layer_forward_ex(dl.desc, x, T, out, ws, mode)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g):
            moe.moe_layer_forward_ex(dl.desc, x, T, out, ws, mode)
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    for r in range(4):
        out.fill_(0)                                            # eager work between replays
        moe.moe_layer_forward_ex(dl.desc, x[: max(1, T // 2)], max(1, T // 2), other, ws, mode)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
