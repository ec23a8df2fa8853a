"""The C-ABI library without a GPU: it loads, exports every function the header
declares, sizes workspaces, and rejects bad arguments on the host (documented
negative codes, nothing enqueued)."""
import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_softmax_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_library_exports_every_declared_function():
    L = moe.lib()
    declared = _declared()
    assert "moe_layer_forward" in declared and "act_quant_nvfp4" in declared
    missing = [n for n in declared if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(moe.EXPORTS) == declared


def test_workspace_sizes():
    L = moe.lib()
    assert L.moe_route_workspace_bytes(8, 512) == 8 * 512 * 4
    assert L.moe_route_workspace_bytes(0, 512) == 0
    # 4-bit mode: x codes/scales per pair and matrix, h codes/scales per pair, work plan
    P, H, I = 80, 3072, 512
    want = sum((n + 255) // 256 * 256
               for n in (P * 2 * H // 2, P * 2 * H // 16, P * I // 2, P * I // 16, (min(P, 1024) + P // 32) * 16))
    assert L.nvfp4_expert_ffn_workspace_bytes(moe.MOE_A4, 8, 10, H, I) == want
    assert L.nvfp4_expert_ffn_workspace_bytes(moe.MOE_A16, 1, 10, H, I) == 10 * I * 2
    assert L.nvfp4_expert_ffn_workspace_bytes(7, 1, 10, H, I) == 0
    assert L.moe_layer_workspace_bytes(moe.MOE_A16, 1, 10, 512, 3072, 500) == 0   # I % 32 != 0
    assert L.moe_layer_workspace_bytes(moe.MOE_A16, 1, 65, 512, 3072, 512) == 0   # k <= 64
    lay = moe.layer_workspace_layout("A4", 1024, 10, 512, 3072, 512)
    # a counter block of the fused decode path comes first, at a fixed place
    assert 0 < lay["topk_ids"] <= 4 << 20 and all(v % 256 == 0 for v in lay.values())


def _err(code):
    return moe.STATUS[code], moe.lib().moe_last_error().decode()


P16 = ctypes.c_void_p(4096)     # aligned non-null host address, never dereferenced
P4 = ctypes.c_void_p(4100)      # 4-byte aligned, not 16


def test_route_validation():
    L = moe.lib()
    assert _err(L.moe_route_topk(None, P16, None, 1, 3072, 512, 10, P16, P16, P16, 1 << 20, None))[0] == "MOE_E_ARG"
    assert _err(L.moe_route_topk(P16, P16, None, 1, 3000, 512, 10, P16, P16, P16, 1 << 20, None))[0] == "MOE_E_SHAPE"
    assert _err(L.moe_route_topk(P16, P16, None, 1, 3072, 512, 513, P16, P16, P16, 1 << 20, None))[0] == "MOE_E_SHAPE"
    assert _err(L.moe_route_topk(P16, P16, None, 1, 3072, 2048, 10, P16, P16, P16, 1 << 30, None))[0] == "MOE_E_SHAPE"
    assert _err(L.moe_route_topk(P4, P16, None, 1, 3072, 512, 10, P16, P16, P16, 1 << 20, None))[0] == "MOE_E_ALIGN"
    code, text = _err(L.moe_route_topk(P16, P16, None, 1, 3072, 512, 10, P16, P16, P16, 16, None))
    assert code == "MOE_E_WORKSPACE" and "workspace" in text


def test_block_launch_query():
    L = moe.lib()
    assert L.moe_block_launches(moe.MOE_A16, 1, 10, 3072, 512, 512) == 1        # shared expert in the one launch
    assert L.moe_block_launches(moe.MOE_A16, 1, 10, 3072, 512, 1024) == 3       # too wide: its own two kernels
    assert L.moe_block_launches(moe.MOE_A4, 8, 10, 3072, 512, 512) == 2 + 2
    assert L.moe_block_launches(moe.MOE_A16, 1024, 10, 3072, 512, 512) == 0     # per-stage path


def test_layer_stage_and_fused_queries():
    L = moe.lib()
    assert L.moe_layer_is_fused(1, 3072, 512) == 1 and L.moe_layer_is_fused(8, 3072, 512) == 1
    assert L.moe_layer_is_fused(9, 3072, 512) == 0          # wider calls: per-stage kernels
    assert L.moe_layer_is_fused(1, 256, 128) == 0           # small H/I: per-stage kernels
    # launches per call: one for 16-bit activations up to 64 pairs, else routing
    # (+ the activation quantizer) + experts, or the per-stage kernels
    assert moe.layer_launches("A16", 1, 10, 3072, 512) == 1
    assert moe.layer_launches("A16", 6, 10, 3072, 512) == 1
    assert moe.layer_launches("A16", 7, 10, 3072, 512) == 2
    assert moe.layer_launches("A8", 2, 10, 3072, 512) == 1   # x quantized in the gate/up tiles
    assert moe.layer_launches("A8", 7, 10, 3072, 512) == 2   # more than 64 pairs: x quantized in the routing kernel
    assert moe.layer_launches("A4", 8, 10, 3072, 512) == 2   # x quantized in the gate/up tiles
    assert moe.layer_launches("A16", 9, 10, 3072, 512) == 0
    assert moe.layer_launches("A16", 1, 2, 256, 128) == 0
    code, text = _err(L.moe_layer_forward_stage(None, 0, 2, P16, P16, None, 1, 2, None, P16, P16, 1 << 20, None))
    assert code == "MOE_E_ARG" and "stage" in text


def test_permute_and_combine_validation():
    L = moe.lib()
    assert _err(L.moe_permute(P16, 1, 10, 5, P16, P16, P16, None, 0, None))[0] == "MOE_E_SHAPE"
    assert _err(L.moe_permute(None, 1, 2, 5, P16, P16, P16, None, 0, None))[0] == "MOE_E_ARG"
    # up to 2048 pairs one workgroup needs no workspace; more pairs need per-block counts
    assert L.moe_permute_workspace_bytes(1, 10, 512) == 0
    assert L.moe_permute_workspace_bytes(204, 10, 512) == 0
    assert L.moe_permute_workspace_bytes(1024, 10, 512) == 10 * 512 * 4
    assert L.moe_permute_workspace_bytes(1025, 10, 512) == 11 * 512 * 4
    code, text = _err(L.moe_permute(P16, 1024, 10, 512, P16, P16, P16, None, 0, None))
    assert code == "MOE_E_WORKSPACE" and "workspace" in text
    assert _err(L.moe_combine(P16, P16, P16, 1, 2, 3000, None, P16, None))[0] == "MOE_E_SHAPE"
    assert _err(L.moe_combine(P16, P16, P16, 1, 2, 3072, ctypes.c_void_p(4098), P16, None))[0] == "MOE_E_ALIGN"


def test_quant_validation():
    L = moe.lib()
    assert _err(L.act_quant_nvfp4(P16, 0, 4, 48, P16, None, P16, P16, None))[0] == "MOE_E_SHAPE"
    assert _err(L.act_quant_nvfp4(P16, 5, 4, 64, P16, None, P16, P16, None))[0] == "MOE_E_ARG"
    assert _err(L.act_quant_fp8(P16, 0, 4, 64, P16, None, None))[0] == "MOE_E_ARG"
    assert _err(L.nvfp4_global_scale(P16, 2, 6, P16, None))[0] == "MOE_E_SHAPE"


def test_expert_validation():
    L = moe.lib()
    s = moe._Experts(4096, 4096, 4096, 4096, 4096, 4096, None, None, 512, 3072, 512)
    args = (P16, 1, 10, P16, P16, P16, P16, 1 << 30, None)
    assert _err(L.nvfp4_expert_ffn(ctypes.byref(s), moe.MOE_A4, *args))[0] == "MOE_E_ARG"  # no inscales
    assert _err(L.nvfp4_expert_ffn(ctypes.byref(s), 9, *args))[0] == "MOE_E_ARG"
    s.I = 500
    assert _err(L.nvfp4_expert_ffn(ctypes.byref(s), moe.MOE_A16, *args))[0] == "MOE_E_SHAPE"
    s.I = 512
    code, _ = _err(L.nvfp4_expert_ffn(ctypes.byref(s), moe.MOE_A16, P16, 1, 10, P16, P16, P16, P16, 100, None))
    assert code == "MOE_E_WORKSPACE"
    assert _err(L.nvfp4_expert_ffn_stage(ctypes.byref(s), moe.MOE_A16, 3, *args))[0] == "MOE_E_ARG"
    out = ctypes.c_void_p(8192)
    assert _err(L.moe_layer_forward(ctypes.byref(s), moe.MOE_A16, P16, P16, None, 1, 10, None, P16,
                                    out, 1 << 30, None))[0] == "MOE_E_ARG"          # out aliases x
    assert _err(L.moe_layer_forward(ctypes.byref(s), moe.MOE_A16, P16, P16, None, 1, 10, None, out,
                                    ctypes.c_void_p(4096 + 16), 1 << 30, None))[0] == "MOE_E_ALIGN"


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        moe.moe_permute(torch.zeros(2, 2, dtype=torch.int32), 4)


def test_debug_matmul_validation():
    """The test-only product core: host-side checks before anything is enqueued."""
    L = moe.lib()
    f = L.moe_debug_nvfp4_matmul
    assert L.moe_debug_nvfp4_matmul_workspace_bytes(0, 40) == 0
    assert L.moe_debug_nvfp4_matmul_workspace_bytes(1, 40) == 2 * 16     # two chunks of <= 32 columns
    assert L.moe_debug_nvfp4_matmul_workspace_bytes(2, 40) == 0
    ok = dict(core=0, mode=moe.MOE_A16, codes=P16, scales=P16, wscale=P16, N=256, K=3072, x=P16,
              x_scales=None, inscale=None, cols=8, out=P16, ws=None, nws=0)

    def call(**kw):
        a = dict(ok, **kw)
        return _err(f(a["core"], a["mode"], a["codes"], a["scales"], a["wscale"], a["N"], a["K"], a["x"],
                      a["x_scales"], a["inscale"], a["cols"], a["out"], a["ws"], a["nws"], None))[0]

    assert call(core=2) == "MOE_E_ARG"
    assert call(mode=5) == "MOE_E_ARG"
    assert call(codes=None) == "MOE_E_ARG"
    assert call(mode=moe.MOE_A8) == "MOE_E_ARG"                          # 8-bit x needs its scales
    assert call(mode=moe.MOE_A4, x_scales=P16) == "MOE_E_ARG"            # 4-bit x needs the input scale
    assert call(K=3000) == "MOE_E_SHAPE"
    assert call(cols=0) == "MOE_E_SHAPE"
    assert call(x=P4) == "MOE_E_ALIGN"
    assert call(core=1, N=250) == "MOE_E_SHAPE"                          # wide core: N % 16
    a4 = dict(mode=moe.MOE_A4, x_scales=P16, inscale=P16)
    assert call(core=1, N=250, **a4) == "MOE_E_SHAPE"                    # N % 16
    assert call(core=1, K=3040, **a4) == "MOE_E_SHAPE"                   # K % 128
    assert call(core=1, **a4) == "MOE_E_WORKSPACE"                       # chunk list needed
    assert call(core=1, ws=P16, nws=8, **a4) == "MOE_E_WORKSPACE"


def test_layer_status_validation():
    L = moe.lib()
    assert _err(L.moe_layer_status(None, None))[0] == "MOE_E_ARG"


def test_layout_and_repack_validation():
    L = moe.lib()
    args = (P16, 1, 10, P16, P16, P16, P16, 1 << 30, None)
    s = moe._Experts(4096, 4096, 4096, 4096, 4096, 4096, None, None, 512, 3072, 512, 0, 7)
    assert _err(L.nvfp4_expert_ffn(ctypes.byref(s), moe.MOE_A16, *args))[0] == "MOE_E_ARG"      # bad layout
    s.layout = moe.LAYOUT_TILED
    s.I = 480                                                                                  # not % 128
    assert _err(L.nvfp4_expert_ffn(ctypes.byref(s), moe.MOE_A16, *args))[0] == "MOE_E_SHAPE"
    s.I, s.fmt = 512, moe.FMT_Q4G64                                                            # tiled is NVFP4 only
    assert _err(L.nvfp4_expert_ffn(ctypes.byref(s), moe.MOE_A16, *args))[0] == "MOE_E_SHAPE"
    src = moe._Experts(1 << 20, 2 << 20, 3 << 20, 4 << 20, 4096, 4096, None, None, 4, 1152, 256, 0, 0)
    dst = moe._Experts(5 << 20, 6 << 20, 7 << 20, 8 << 20, 4096, 4096, None, None, 4, 1152, 256, 0, 1)
    assert _err(L.moe_nvfp4_repack(None, ctypes.byref(dst), None))[0] == "MOE_E_ARG"
    dst.layout = 0
    assert _err(L.moe_nvfp4_repack(ctypes.byref(src), ctypes.byref(dst), None))[0] == "MOE_E_ARG"   # dst not tiled
    dst.layout, dst.H = 1, 1024
    assert _err(L.moe_nvfp4_repack(ctypes.byref(src), ctypes.byref(dst), None))[0] == "MOE_E_SHAPE"  # shapes differ
    dst.H, src.I, dst.I = 1152, 224, 224
    assert _err(L.moe_nvfp4_repack(ctypes.byref(src), ctypes.byref(dst), None))[0] == "MOE_E_SHAPE"  # I % 128
    src.I = dst.I = 256
    dst.gu_scales = src.gu_scales + 64                                                         # overlapping scales
    assert _err(L.moe_nvfp4_repack(ctypes.byref(src), ctypes.byref(dst), None))[0] == "MOE_E_ARG"
    dst.gu_scales = (6 << 20) + 8
    assert _err(L.moe_nvfp4_repack(ctypes.byref(src), ctypes.byref(dst), None))[0] == "MOE_E_ALIGN"
