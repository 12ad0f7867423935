"""The C ABI on the CPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import quantized_moe_expert_02_amd as moe
from quantized_moe_expert_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 9
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(_lib.EXPORTED)
    assert moe.moe_abi_version() == 1


FAKE = 1 << 20  # a 256-byte aligned non-null address; never dereferenced


def qw(fmt, E, rows, cols):
    q = _lib.moe_qweight()
    q.format, q.rows, q.cols, q.num_experts = fmt, rows, cols, E
    q.codes = FAKE
    q.scales = FAKE
    q.tensor_scale = FAKE if fmt == moe.MOE_FMT_NVFP4 else None
    rb = cols if fmt == moe.MOE_FMT_FP8_B128 else cols // 2
    q.expert_stride_codes = rows * rb
    if fmt == moe.MOE_FMT_NVFP4:
        q.expert_stride_scales = rows * cols // 16
    elif fmt == moe.MOE_FMT_MXFP4:
        q.expert_stride_scales = rows * cols // 32
    else:
        q.expert_stride_scales = ((rows + 127) // 128) * ((cols + 127) // 128) * 4
    return q


def layer(fmt=1, H=2048, I=512, E=512, k=10, shared=True):
    L = _lib.moe_layer_desc()
    L.H, L.I, L.E, L.top_k, L.renormalize = H, I, E, k, 1
    L.router_w = FAKE
    L.gate, L.up, L.down = qw(fmt, E, I, H), qw(fmt, E, I, H), qw(fmt, E, H, I)
    if shared:
        L.has_shared, L.I_shared = 1, 512
        f8 = moe.MOE_FMT_FP8_B128
        L.sh_gate, L.sh_up, L.sh_down = qw(f8, 1, 512, H), qw(f8, 1, 512, H), qw(f8, 1, H, 512)
    return L


def test_valid_descriptors_for_every_format():
    for fmt in (1, 2, 3):
        L = layer(fmt)
        assert moe.moe_validate_layer(L) == moe.MOE_OK
        assert moe.moe_workspace_size(L, 8) > 0
        assert moe.moe_workspace_size(L, 8192) > moe.moe_workspace_size(L, 8)


@pytest.mark.parametrize("mutate,code", [
    (lambda L: setattr(L, "top_k", 600), -1),
    (lambda L: setattr(L, "top_k", 0), -1),
    (lambda L: setattr(L, "top_k", 40), -2),
    (lambda L: setattr(L, "renormalize", 2), -1),
    (lambda L: setattr(L, "router_w", None), -1),
    (lambda L: setattr(L.gate, "format", 9), -2),
    (lambda L: setattr(L.gate, "rows", 500), -1),
    (lambda L: setattr(L.down, "codes", FAKE + 8), -1),
    (lambda L: setattr(L.down, "tensor_scale", None), -1),
    (lambda L: setattr(L.up, "expert_stride_codes", 16), -1),
    (lambda L: setattr(L.sh_down, "num_experts", 2), -1),
    (lambda L: setattr(L, "I_shared", 0), -1),
])
def test_bad_descriptor_rejected(mutate, code):
    L = layer()
    mutate(L)
    assert moe.moe_validate_layer(L) == code
    assert moe.moe_workspace_size(L, 1) == 0


def test_unaligned_or_odd_shapes_unsupported():
    L = layer(1, H=2048 + 16)         # NVFP4 K not a multiple of 32
    L.has_shared = 0
    assert moe.moe_validate_layer(L) == moe.MOE_ERR_UNSUPPORTED
    L = layer(3, H=2048 + 16, shared=False)   # FP8 K multiple of 16 is fine
    assert moe.moe_validate_layer(L) == moe.MOE_OK
    L = layer(2, E=2048, shared=False)
    assert moe.moe_validate_layer(L) == moe.MOE_ERR_UNSUPPORTED


def test_entry_points_reject_before_any_launch():
    L = layer()
    st = moe.moe_layer_forward(L, FAKE, 4, FAKE, FAKE, 16, check=False)
    assert st == moe.MOE_ERR_WORKSPACE
    st = moe.moe_layer_forward(L, FAKE + 2, 4, FAKE, FAKE, 1 << 40, check=False)
    assert st == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_layer_forward(L, None, 0, None, None, 0, check=False) == moe.MOE_OK
    assert moe.moe_layer_forward(L, FAKE, -1, FAKE, FAKE, 0, check=False) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_route_topk(L, FAKE, FAKE, 4, FAKE, FAKE, None, 0, check=False) == moe.MOE_ERR_WORKSPACE
    assert moe.moe_route_topk(L, None, None, 4, FAKE, FAKE, None, 0, check=False) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_permute(FAKE, 4, 11, 10, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, check=False) == -1
    assert moe.moe_permute(FAKE, 4, 2, 10, FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, check=False) == -3
    assert moe.moe_combine(FAKE, FAKE, FAKE, None, 4, 2, 2050, FAKE, check=False) == -2
    assert moe.moe_expert_gemm(7, L, 0, FAKE, FAKE, None, 4, FAKE, FAKE, FAKE, 1 << 40, check=False) == -1
    L.has_shared = 0
    assert moe.moe_expert_gemm(0, L, 1, None, None, None, 4, FAKE, FAKE, None, 0, check=False) == -1


def test_noalloc_entry_point_rejects_sizes_beyond_its_array():
    """moe_layer_forward_noalloc: host-side checks only (no GPU here); a T
    whose workspace exceeds the fixed array is refused before any HIP call."""
    L = layer()
    limit = moe.moe_noalloc_workspace_limit()
    assert limit == 32 << 20
    T_big = 1
    while moe.moe_workspace_size(L, T_big) <= limit:
        T_big *= 2
    assert moe.moe_layer_forward_noalloc(L, FAKE, T_big, FAKE, check=False) == moe.MOE_ERR_WORKSPACE
    assert moe.moe_layer_forward_noalloc(L, None, 0, None, check=False) == moe.MOE_OK
    assert moe.moe_layer_forward_noalloc(L, FAKE + 2, 4, FAKE, check=False) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_layer_forward_noalloc(L, FAKE, -1, FAKE, check=False) == moe.MOE_ERR_INVALID_ARG


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    import importlib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libmoe.so"))
    with pytest.raises(ImportError):
        _lib._load()
