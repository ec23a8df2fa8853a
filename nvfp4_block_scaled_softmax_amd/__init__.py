"""Python binding of libmoe_nvfp4.so, the NVFP4 routed-expert layer for MI355X.

Argument marshalling only: every function checks dtypes, shapes, devices and
contiguity of torch tensors, allocates the outputs with torch, and calls the
C entry point of the same name on the current torch stream.  Every step of the
layer runs in the library's HIP kernels; there is no fallback.  The C ABI and
its semantics are documented in include/moe_nvfp4.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_NVFP4_LIB names another build of the same sources (the host-sanitizer
# build of sanitize.py); by default the in-tree library.
LIB_PATH = os.environ.get("MOE_NVFP4_LIB") or os.path.join(_HERE, "libmoe_nvfp4.so")

MOE_A16, MOE_A8, MOE_A4 = 0, 1, 2
MODES = {"A16": MOE_A16, "A8": MOE_A8, "A4": MOE_A4,
         "F16": MOE_A16}   # "F16": the 16-bit activations as q4_g64_fp16 experts take them (fp16)
DT_BF16, DT_F32 = 0, 1
FMT_NVFP4, FMT_Q4G64 = 0, 2
LAYOUT_CANONICAL, LAYOUT_TILED = 0, 1
STATUS = {0: "MOE_OK", -1: "MOE_E_ARG", -2: "MOE_E_ALIGN", -3: "MOE_E_SHAPE",
          -4: "MOE_E_UNSUPPORTED", -5: "MOE_E_WORKSPACE", -6: "MOE_E_HIP", -7: "MOE_E_STALLED"}

EXPORTS = ("moe_last_error", "moe_route_workspace_bytes", "moe_route_topk",
           "moe_permute_workspace_bytes", "moe_permute",
           "act_quant_nvfp4", "act_quant_fp8", "nvfp4_global_scale",
           "nvfp4_expert_ffn_workspace_bytes", "nvfp4_expert_ffn", "nvfp4_expert_ffn_stage",
           "moe_combine",
           "moe_layer_workspace_bytes", "moe_layer_workspace_layout", "moe_layer_wait_timeouts_offset",
           "moe_layer_forward", "moe_layer_forward_stage", "moe_layer_is_fused", "moe_layer_launches", "moe_block_launches",
           "moe_layer_status", "moe_debug_nvfp4_matmul_workspace_bytes", "moe_debug_nvfp4_matmul",
           "moe_layer_forward_noalloc",
           "moe_shared_expert_workspace_bytes", "moe_shared_expert_forward", "moe_combine_shared",
           "moe_block_workspace_bytes", "moe_block_workspace_layout", "moe_block_forward",
           "q4g64_quantize", "moe_debug_q4g64_matmul", "moe_nvfp4_repack")


class MoeError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__(f"{fn}: {STATUS.get(code, code)}: {text}")
        self.code = code


class _Experts(ctypes.Structure):
    _fields_ = [("gu_codes", ctypes.c_void_p), ("gu_scales", ctypes.c_void_p),
                ("dn_codes", ctypes.c_void_p), ("dn_scales", ctypes.c_void_p),
                ("gu_wscale", ctypes.c_void_p), ("dn_wscale", ctypes.c_void_p),
                ("gu_inscale", ctypes.c_void_p), ("dn_inscale", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("fmt", ctypes.c_int32), ("layout", ctypes.c_int32)]


class _Shared(ctypes.Structure):
    _fields_ = [("gu", ctypes.c_void_p), ("dn", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("H", ctypes.c_int32), ("Is", ctypes.c_int32)]


_lib = None
_P, _I, _Z, _L = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int64


def lib():
    """The loaded library; raises if it is not built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                               "python -m nvfp4_block_scaled_softmax_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_last_error": ([], ctypes.c_char_p),
            "moe_route_workspace_bytes": ([_I, _I], _Z),
            "moe_route_topk": ([_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
            "moe_permute_workspace_bytes": ([_I, _I, _I], _Z),
            "moe_permute": ([_P, _I, _I, _I, _P, _P, _P, _P, _Z, _P], _I),
            "act_quant_nvfp4": ([_P, _I, _I, _I, _P, _P, _P, _P, _P], _I),
            "act_quant_fp8": ([_P, _I, _I, _I, _P, _P, _P], _I),
            "nvfp4_global_scale": ([_P, _I, _L, _P, _P], _I),
            "nvfp4_expert_ffn_workspace_bytes": ([_I, _I, _I, _I, _I], _Z),
            "nvfp4_expert_ffn": ([ctypes.POINTER(_Experts), _I, _P, _I, _I, _P, _P, _P, _P, _Z, _P], _I),
            "nvfp4_expert_ffn_stage": ([ctypes.POINTER(_Experts), _I, _I, _P, _I, _I, _P, _P, _P, _P, _Z, _P], _I),
            "moe_combine": ([_P, _P, _P, _I, _I, _I, _P, _P, _P], _I),
            "moe_layer_workspace_bytes": ([_I, _I, _I, _I, _I, _I], _Z),
            "moe_layer_workspace_layout": ([_I, _I, _I, _I, _I, _I, ctypes.POINTER(_Z)], _I),
            "moe_layer_wait_timeouts_offset": ([], _Z),
            "moe_layer_is_fused": ([_I, _I, _I], _I),
            "moe_layer_launches": ([_I, _I, _I, _I, _I], _I),
            "moe_block_launches": ([_I, _I, _I, _I, _I, _I], _I),
            "moe_layer_forward_stage": ([ctypes.POINTER(_Experts), _I, _I, _P, _P, _P, _I, _I, _P, _P, _P, _Z, _P], _I),
            "moe_layer_forward": ([ctypes.POINTER(_Experts), _I, _P, _P, _P, _I, _I, _P, _P, _P, _Z, _P], _I),
            "moe_layer_status": ([_P, _P], _I),
            "q4g64_quantize": ([_P, _I, _I, _P, _P, _P], _I),
            "moe_debug_q4g64_matmul": ([_P, _P, _I, _I, _P, _I, _P, _P], _I),
            "moe_nvfp4_repack": ([ctypes.POINTER(_Experts), ctypes.POINTER(_Experts), _P], _I),
            "moe_shared_expert_workspace_bytes": ([_I, _I], _Z),
            "moe_shared_expert_forward": ([ctypes.POINTER(_Shared), _P, _I, _P, _P, _Z, _P], _I),
            "moe_combine_shared": ([_P, _P, _P, _I, _I, _I, _P, _P, _P, _P], _I),
            "moe_block_workspace_bytes": ([_I, _I, _I, _I, _I, _I, _I], _Z),
            "moe_block_workspace_layout": ([_I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_Z)], _I),
            "moe_block_forward": ([ctypes.POINTER(_Experts), ctypes.POINTER(_Shared), _I, _P, _P, _P, _I, _I, _P,
                                   _P, _P, _Z, _P], _I),
            "moe_layer_forward_noalloc": ([ctypes.POINTER(_Experts), _I, _P, _P, _P, _I, _I, _P, _P, _I, _P], _I),
            "moe_debug_nvfp4_matmul_workspace_bytes": ([_I, _I], _Z),
            "moe_debug_nvfp4_matmul": ([_I, _I, _P, _P, _P, _I, _I, _P, _P, _P, _I, _P, _P, _Z, _P], _I),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(fn, code):
    if code != 0:
        raise MoeError(fn, code, lib().moe_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _bf16(t, name):
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError(f"{name}: expected bfloat16 (or its 16-bit patterns), got {t.dtype}")


def _mode(mode):
    return MODES[mode] if isinstance(mode, str) else int(mode)


# --------------------------------------------------------------------------- experts
@dataclasses.dataclass
class Experts:
    """One layer's experts on the GPU (see the C header).  NVFP4 (fmt FMT_NVFP4)
    or q4_g64_fp16 (fmt FMT_Q4G64: scales fp16 bits, one per 64, no
    multipliers); layout LAYOUT_CANONICAL, or LAYOUT_TILED (NVFP4 scales
    rearranged by moe_nvfp4_repack)."""
    gu_codes: torch.Tensor     # uint8 [E, 2I, H/2]
    gu_scales: torch.Tensor    # uint8 [E, 2I, H/16]  (q4: 16-bit [E, 2I, H/64])
    dn_codes: torch.Tensor     # uint8 [E, H, I/2]
    dn_scales: torch.Tensor    # uint8 [E, H, I/16]   (q4: 16-bit [E, H, I/64])
    gu_wscale: torch.Tensor | None = None    # float32 [E, 2] (NVFP4)
    dn_wscale: torch.Tensor | None = None    # float32 [E] (NVFP4)
    gu_inscale: torch.Tensor | None = None   # float32 [E, 2]
    dn_inscale: torch.Tensor | None = None   # float32 [E]
    fmt: int = 0
    layout: int = 0

    @property
    def E(self):
        return self.gu_codes.shape[0]

    @property
    def H(self):
        return self.dn_codes.shape[1]

    @property
    def I(self):
        return self.gu_codes.shape[1] // 2

    def struct(self):
        """The C struct (validated once, then cached: the tensors must not be replaced)."""
        cached = self.__dict__.get("_cstruct")
        if cached is not None:
            return cached
        E, H, I = self.E, self.H, self.I
        _need(self.gu_codes, "gu_codes", torch.uint8, (E, 2 * I, H // 2))
        _need(self.dn_codes, "dn_codes", torch.uint8, (E, H, I // 2))
        if self.fmt == FMT_Q4G64:
            for n, t, shp in (("gu_scales", self.gu_scales, (E, 2 * I, H // 64)),
                              ("dn_scales", self.dn_scales, (E, H, I // 64))):
                _need(t, n, shape=shp)
                if t.element_size() != 2:
                    raise TypeError(f"{n}: q4_g64_fp16 scales are 16-bit, got {t.dtype}")
        else:
            _need(self.gu_scales, "gu_scales", torch.uint8, (E, 2 * I, H // 16))
            _need(self.dn_scales, "dn_scales", torch.uint8, (E, H, I // 16))
            _need(self.gu_wscale, "gu_wscale", torch.float32, (E, 2))
            _need(self.dn_wscale, "dn_wscale", torch.float32, (E,))
        if self.gu_inscale is not None:
            _need(self.gu_inscale, "gu_inscale", torch.float32, (E, 2))
        if self.dn_inscale is not None:
            _need(self.dn_inscale, "dn_inscale", torch.float32, (E,))
        opt = lambda t: None if t is None else t.data_ptr()
        st = _Experts(self.gu_codes.data_ptr(), self.gu_scales.data_ptr(),
                      self.dn_codes.data_ptr(), self.dn_scales.data_ptr(),
                      opt(self.gu_wscale), opt(self.dn_wscale), opt(self.gu_inscale), opt(self.dn_inscale),
                      E, H, I, int(self.fmt), int(self.layout))
        self.__dict__["_cstruct"] = st
        return st


@dataclasses.dataclass
class SharedExpert:
    """A layer's BF16 shared expert on the GPU (see moe_shared_expert in the C header)."""
    gu: torch.Tensor      # bf16 [2Is, H]: gate rows, then up rows
    dn: torch.Tensor      # bf16 [H, Is]
    gate: torch.Tensor    # bf16 [H]

    @property
    def H(self):
        return self.dn.shape[0]

    @property
    def Is(self):
        return self.dn.shape[1]

    def struct(self):
        cached = self.__dict__.get("_cstruct")
        if cached is not None:
            return cached
        H, Is = self.H, self.Is
        for name, t, shape in (("gu", self.gu, (2 * Is, H)), ("dn", self.dn, (H, Is)), ("gate", self.gate, (H,))):
            _need(_bf16(t, name), name, shape=shape)
        st = _Shared(self.gu.data_ptr(), self.dn.data_ptr(), self.gate.data_ptr(), H, Is)
        self.__dict__["_cstruct"] = st
        return st


# --------------------------------------------------------------------------- entry points
def moe_route_topk(x, w_router, k, bias=None, ids=None, w=None, ws=None):
    """Router logits, softmax, top-k, renormalise.  Returns (ids int32 [T,k], w fp32 [T,k]).

    ids / w / ws may be given (preallocated) to avoid allocations."""
    x, w_router = _bf16(x, "x"), _bf16(w_router, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, "x")
    _need(w_router, "w_router", shape=(E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    if ids is None:
        ids = torch.empty(T, k, dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty(T, k, dtype=torch.float32, device=x.device)
    _need(ids, "ids", torch.int32, (T, k))
    _need(w, "w", torch.float32, (T, k))
    nws = lib().moe_route_workspace_bytes(T, E)
    if ws is None:
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=x.device)
    _check("moe_route_topk", lib().moe_route_topk(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k,
                                                  _ptr(ids), _ptr(w), _ptr(ws), ws.numel(),
                                                  _stream()))
    return ids, w


def moe_permute(topk_ids, E, off=None, sp=None, pr=None, ws=None):
    """Returns (expert_offsets [E+1], sorted_pairs [T*k], pair_row [T*k]), all int32."""
    _need(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    dev = topk_ids.device
    off = torch.empty(E + 1, dtype=torch.int32, device=dev) if off is None else off
    sp = torch.empty(T * k, dtype=torch.int32, device=dev) if sp is None else sp
    pr = torch.empty(T * k, dtype=torch.int32, device=dev) if pr is None else pr
    _need(off, "expert_offsets", torch.int32, (E + 1,))
    _need(sp, "sorted_pairs", torch.int32, (T * k,))
    _need(pr, "pair_row", torch.int32, (T * k,))
    need = lib().moe_permute_workspace_bytes(T, k, E)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("moe_permute", lib().moe_permute(_ptr(topk_ids), T, k, E, _ptr(off), _ptr(sp), _ptr(pr),
                                            _ptr(ws) if ws is not None else None,
                                            ws.numel() if ws is not None else 0, _stream()))
    return off, sp, pr


def act_quant_nvfp4(x, global_scale, row_group=None):
    """NVFP4 per 16 along rows of x (bf16 or fp32).  Returns (codes [R, C/2], scales [R, C/16])."""
    _need(x, "x")
    dt = DT_F32 if x.dtype == torch.float32 else DT_BF16
    if dt == DT_BF16:
        _bf16(x, "x")
    R, C = x.shape
    _need(global_scale, "global_scale", torch.float32)
    if row_group is not None:
        _need(row_group, "row_group", torch.int32, (R,))
    codes = torch.empty(R, C // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(R, C // 16, dtype=torch.uint8, device=x.device)
    _check("act_quant_nvfp4", lib().act_quant_nvfp4(_ptr(x), dt, R, C, _ptr(global_scale),
                                                    _ptr(row_group), _ptr(codes), _ptr(scales),
                                                    _stream()))
    return codes, scales


def act_quant_fp8(x):
    """8-bit mode per 16 along rows.  Returns (E4M3 codes [R, C], fp32 scales [R, C/16])."""
    _need(x, "x")
    dt = DT_F32 if x.dtype == torch.float32 else DT_BF16
    if dt == DT_BF16:
        _bf16(x, "x")
    R, C = x.shape
    codes = torch.empty(R, C, dtype=torch.uint8, device=x.device)
    scales = torch.empty(R, C // 16, dtype=torch.float32, device=x.device)
    _check("act_quant_fp8", lib().act_quant_fp8(_ptr(x), dt, R, C, _ptr(codes), _ptr(scales),
                                                _stream()))
    return codes, scales


def q4g64_quantize(x):
    """q4_g64_fp16 packing of fp32 rows x [R, C] (C % 64 == 0).  Returns (codes uint8
    [R, C/2], scales int16 [R, C/64] holding fp16 bit patterns)."""
    _need(x, "x", torch.float32)
    R, C = x.shape
    codes = torch.empty(R, C // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(R, C // 64, dtype=torch.int16, device=x.device)
    _check("q4g64_quantize", lib().q4g64_quantize(_ptr(x), R, C, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def moe_nvfp4_repack(experts: Experts, share_codes=True):
    """The experts in the tiled layout (moe_nvfp4_repack): new scale arrays, the
    codes shared with `experts` (or copies, share_codes=False), the fp32 arrays
    shared."""
    src = experts.struct()
    tiled = dataclasses.replace(experts, layout=LAYOUT_TILED,
                                gu_codes=experts.gu_codes if share_codes else torch.empty_like(experts.gu_codes),
                                dn_codes=experts.dn_codes if share_codes else torch.empty_like(experts.dn_codes),
                                gu_scales=torch.empty_like(experts.gu_scales),
                                dn_scales=torch.empty_like(experts.dn_scales))
    tiled.__dict__.pop("_cstruct", None)
    _check("moe_nvfp4_repack", lib().moe_nvfp4_repack(ctypes.byref(src), ctypes.byref(tiled.struct()), _stream()))
    return tiled


def pack_experts_q4(w_gu, w_dn):
    """q4_g64_fp16-pack fp32 expert weights on the GPU: w_gu [E, 2I, H] (gate rows then
    up rows), w_dn [E, H, I]."""
    _need(w_gu, "w_gu", torch.float32)
    _need(w_dn, "w_dn", torch.float32)
    E, I2, H = w_gu.shape
    I = I2 // 2
    gc, gs = q4g64_quantize(w_gu.view(E * 2 * I, H))
    dc, ds = q4g64_quantize(w_dn.view(E * H, I))
    return Experts(gc.view(E, 2 * I, H // 2), gs.view(E, 2 * I, H // 64), dc.view(E, H, I // 2),
                   ds.view(E, H, I // 64), fmt=FMT_Q4G64)


def debug_q4g64_matmul(codes, scales, x16, out=None):
    """Test-only: the q4_g64_fp16 narrow core, out [cols, N] fp32 = x16 . dequant(W)^T
    (x16: fp16 [cols, K], as the experts take it)."""
    N, K2 = codes.shape
    K = 2 * K2
    _need(codes, "codes", torch.uint8, (N, K // 2))
    _need(scales, "scales", shape=(N, K // 64))
    _need(x16, "x16", torch.float16)
    cols = x16.shape[0]
    if out is None:
        out = torch.empty(cols, N, dtype=torch.float32, device=codes.device)
    _check("moe_debug_q4g64_matmul", lib().moe_debug_q4g64_matmul(_ptr(codes), _ptr(scales), N, K, _ptr(x16), cols,
                                                                  _ptr(out), _stream()))
    return out


def nvfp4_global_scale(x):
    """Per-matrix multiplier f32(amax / 2688) of x [n_mat, ...] fp32."""
    _need(x, "x", torch.float32)
    n = x.shape[0]
    g = torch.empty(n, dtype=torch.float32, device=x.device)
    _check("nvfp4_global_scale", lib().nvfp4_global_scale(_ptr(x), n, x.numel() // n, _ptr(g),
                                                          _stream()))
    return g


def ffn_workspace_bytes(mode, T, k, H, I):
    return lib().nvfp4_expert_ffn_workspace_bytes(_mode(mode), T, k, H, I)


def nvfp4_expert_ffn(experts: Experts, mode, x, k, expert_offsets, sorted_pairs, ws=None):
    """Every pair's SwiGLU expert in sorted order.  Returns (y_pairs fp32 [T*k, H], workspace)."""
    x = _bf16(x, "x")
    _need(x, "x")
    T, H = x.shape
    s = experts.struct()
    m = _mode(mode)
    nws = ffn_workspace_bytes(m, T, k, H, experts.I)
    if ws is None:
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=x.device)
    y = torch.empty(T * k, H, dtype=torch.float32, device=x.device)
    _check("nvfp4_expert_ffn", lib().nvfp4_expert_ffn(ctypes.byref(s), m, _ptr(x), T, k,
                                                      _ptr(expert_offsets), _ptr(sorted_pairs),
                                                      _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y, ws


def nvfp4_expert_ffn_stage(experts: Experts, mode, stage, x, k, expert_offsets, sorted_pairs, y,
                           ws):
    """One stage (0 quantize x, 1 gate/up + SwiGLU, 2 down) of nvfp4_expert_ffn, in place."""
    x = _bf16(x, "x")
    _need(x, "x")
    T, H = x.shape
    s = experts.struct()
    _check("nvfp4_expert_ffn_stage",
           lib().nvfp4_expert_ffn_stage(ctypes.byref(s), _mode(mode), stage, _ptr(x), T, k,
                                        _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(y), _ptr(ws),
                                        ws.numel(), _stream()))


def moe_combine(y_pairs, pair_row, topk_w, residual=None, out=None):
    """bf16 output [T, H] (bf16(x + out) when residual is given), as int16 bit patterns."""
    _need(y_pairs, "y_pairs", torch.float32)
    _need(topk_w, "topk_w", torch.float32)
    T, k = topk_w.shape
    H = y_pairs.shape[1]
    _need(pair_row, "pair_row", torch.int32, (T * k,))
    if residual is not None:
        residual = _bf16(residual, "residual")
        _need(residual, "residual")
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=y_pairs.device)
    _need(out, "out", shape=(T, H))
    _check("moe_combine", lib().moe_combine(_ptr(y_pairs), _ptr(pair_row), _ptr(topk_w), T, k, H,
                                            _ptr(residual), _ptr(out), _stream()))
    return out


def moe_shared_expert_forward(shared: SharedExpert, x, ws=None, y=None):
    """The shared expert's gated output, fp32 [T, H].  Returns (y, workspace); the
    workspace holds its bf16 intermediate [T, Is]."""
    x = _bf16(x, "x")
    _need(x, "x")
    T, H = x.shape
    st = shared.struct()
    n = lib().moe_shared_expert_workspace_bytes(T, shared.Is)
    if ws is None:
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty(T, H, dtype=torch.float32, device=x.device)
    _check("moe_shared_expert_forward",
           lib().moe_shared_expert_forward(ctypes.byref(st), _ptr(x), T, _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y, ws


def moe_combine_shared(y_pairs, pair_row, topk_w, shared_y, residual=None, out=None):
    """moe_combine with the shared expert's gated output added before the rounding."""
    _need(y_pairs, "y_pairs", torch.float32)
    _need(topk_w, "topk_w", torch.float32)
    T, k = topk_w.shape
    H = y_pairs.shape[1]
    _need(pair_row, "pair_row", torch.int32, (T * k,))
    _need(shared_y, "shared_y", torch.float32, (T, H))
    if residual is not None:
        residual = _bf16(residual, "residual")
        _need(residual, "residual")
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=y_pairs.device)
    _check("moe_combine_shared", lib().moe_combine_shared(_ptr(y_pairs), _ptr(pair_row), _ptr(topk_w), T, k, H,
                                                          _ptr(shared_y), _ptr(residual), _ptr(out), _stream()))
    return out


def block_workspace_bytes(mode, T, k, E, H, I, Is):
    return lib().moe_block_workspace_bytes(_mode(mode), T, k, E, H, I, Is)


def block_workspace_views(ws, mode, T, k, E, H, I, Is):
    """workspace_views of a block workspace plus the shared expert's intermediate and output."""
    offs = (ctypes.c_size_t * 9)()
    _check("moe_block_workspace_layout", lib().moe_block_workspace_layout(_mode(mode), T, k, E, H, I, Is, offs))
    v = workspace_views(ws, mode, T, k, E, H, I)
    v["shared_h"] = ws[offs[7]:offs[7] + T * Is * 2].view(torch.bfloat16).view(T, Is)
    v["shared_y"] = ws[offs[8]:offs[8] + T * H * 4].view(torch.float32).view(T, H)
    return v


def moe_block_forward(experts: Experts, shared: SharedExpert, mode, x, w_router, k, bias=None, residual=None,
                      ws=None, out=None):
    """The layer with its shared expert.  Returns (out bf16 [T, H], workspace); a
    workspace passed in must have been zero-filled before its first use."""
    x = _bf16(x, "x")
    _need(x, "x")
    T, H = x.shape
    s = experts.struct()
    sh = shared.struct()
    m = _mode(mode)
    w_router = _bf16(w_router, "w_router")
    _need(w_router, "w_router", shape=(experts.E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (experts.E,))
    if residual is not None:
        residual = _bf16(residual, "residual")
        _need(residual, "residual", shape=(T, H))
    nws = block_workspace_bytes(m, T, k, experts.E, H, experts.I, shared.Is)
    if ws is None:
        ws = torch.zeros(max(nws, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    _check("moe_block_forward", lib().moe_block_forward(ctypes.byref(s), ctypes.byref(sh), m, _ptr(x),
                                                        _ptr(w_router), _ptr(bias), T, k, _ptr(residual), _ptr(out),
                                                        _ptr(ws), ws.numel(), _stream()))
    return out, ws


def layer_workspace_bytes(mode, T, k, E, H, I):
    return lib().moe_layer_workspace_bytes(_mode(mode), T, k, E, H, I)


def layer_workspace_layout(mode, T, k, E, H, I):
    offs = (ctypes.c_size_t * 7)()
    _check("moe_layer_workspace_layout",
           lib().moe_layer_workspace_layout(_mode(mode), T, k, E, H, I, offs))
    names = ("topk_ids", "topk_w", "expert_offsets", "sorted_pairs", "pair_row", "y_pairs", "ffn")
    return dict(zip(names, list(offs)))


def moe_layer_forward(experts: Experts, mode, x, w_router, k, bias=None, residual=None, ws=None,
                      out=None):
    """The whole layer on the current stream.  Returns (out bf16 [T, H], workspace).
    A workspace passed in must have been zero-filled before its first use (the
    library leaves it ready for the next call)."""
    x = _bf16(x, "x")
    _need(x, "x")
    T, H = x.shape
    s = experts.struct()
    m = _mode(mode)
    w_router = _bf16(w_router, "w_router")
    _need(w_router, "w_router", shape=(experts.E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (experts.E,))
    if residual is not None:
        residual = _bf16(residual, "residual")
        _need(residual, "residual", shape=(T, H))
    nws = layer_workspace_bytes(m, T, k, experts.E, H, experts.I)
    if ws is None:
        ws = torch.zeros(max(nws, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    _check("moe_layer_forward", lib().moe_layer_forward(ctypes.byref(s), m, _ptr(x), _ptr(w_router),
                                                        _ptr(bias), T, k, _ptr(residual), _ptr(out),
                                                        _ptr(ws), ws.numel(), _stream()))
    return out, ws


NOALLOC_SCRATCH_BYTES = 16 << 20


def moe_layer_forward_noalloc(experts: Experts, mode, x, w_router, k, bias=None, residual=None, out=None,
                              reset=False):
    """moe_layer_forward on the library's own device scratch (no workspace argument;
    the C call allocates nothing).  Calls on one GPU must not overlap.  Returns out."""
    x = _bf16(x, "x")
    _need(x, "x")
    T, H = x.shape
    s = experts.struct()
    w_router = _bf16(w_router, "w_router")
    _need(w_router, "w_router", shape=(experts.E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (experts.E,))
    if residual is not None:
        residual = _bf16(residual, "residual")
        _need(residual, "residual", shape=(T, H))
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", shape=(T, H))
    _check("moe_layer_forward_noalloc",
           lib().moe_layer_forward_noalloc(ctypes.byref(s), _mode(mode), _ptr(x), _ptr(w_router), _ptr(bias), T, k,
                                           _ptr(residual), _ptr(out), 1 if reset else 0, _stream()))
    return out


def moe_layer_forward_stage(experts: Experts, mode, stage, x, w_router, k, bias, residual, ws, out):
    """One half (0 routing, 1 experts + combine) of moe_layer_forward, in place."""
    m = _mode(mode)
    T = x.shape[0]
    s = experts.struct()
    _check("moe_layer_forward_stage",
           lib().moe_layer_forward_stage(ctypes.byref(s), m, stage, _ptr(x), _ptr(w_router), _ptr(bias), T,
                                         k, _ptr(residual), _ptr(out), _ptr(ws), ws.numel(), _stream()))


def layer_launches(mode, T, k, H, I):
    """Kernel launches of one moe_layer_forward call outside graph capture (0: per-stage path)."""
    return int(lib().moe_layer_launches(_mode(mode), T, k, H, I))


def block_launches(mode, T, k, H, I, Is):
    """Kernel launches of one moe_block_forward call (1: the shared expert runs in the
    single decode launch; 0: per-stage path)."""
    return int(lib().moe_block_launches(_mode(mode), T, k, H, I, Is))


def layer_wait_timeouts(ws):
    """Waits of the fused decode path that gave up (0 in correct operation)."""
    o = lib().moe_layer_wait_timeouts_offset()
    return int(ws[o:o + 4].view(torch.int32).item())


def moe_layer_status(ws):
    """Raises MoeError (MOE_E_STALLED) when a fused decode wait on this workspace gave
    up since it was zero-filled.  Synchronises the current stream."""
    _need(ws, "ws", torch.uint8)
    _check("moe_layer_status", lib().moe_layer_status(_ptr(ws), _stream()))


def debug_nvfp4_matmul(core, mode, codes, scales, wscale, x, x_scales=None, inscale=None, out=None):
    """Test-only: the expert kernels' product core, out [cols, N] fp32 =
    wscale (* inscale) * x . dequant(W)^T (see moe_debug_nvfp4_matmul in the C header).
    core 0 narrow tile, 1 wide matrix-core loop.  codes uint8 [N, K/2], scales uint8
    [N, K/16], wscale / inscale fp32 [1] device tensors; x per mode: bf16 [cols, K],
    uint8 E4M3 [cols, K] (+ fp32 x_scales [cols, K/16]) or uint8 E2M1 [cols, K/2]
    (+ uint8 x_scales [cols, K/16])."""
    m = _mode(mode)
    N, K2 = codes.shape
    K = 2 * K2
    _need(codes, "codes", torch.uint8, (N, K // 2))
    _need(scales, "scales", torch.uint8, (N, K // 16))
    _need(wscale, "wscale", torch.float32)
    cols = x.shape[0]
    if m == MOE_A16:
        x = _bf16(x, "x")
        _need(x, "x", shape=(cols, K))
    elif m == MOE_A8:
        _need(x, "x", torch.uint8, (cols, K))
        _need(x_scales, "x_scales", torch.float32, (cols, K // 16))
    else:
        _need(x, "x", torch.uint8, (cols, K // 2))
        _need(x_scales, "x_scales", torch.uint8, (cols, K // 16))
        _need(inscale, "inscale", torch.float32)
    if out is None:
        out = torch.empty(cols, N, dtype=torch.float32, device=codes.device)
    _need(out, "out", torch.float32, (cols, N))
    nws = lib().moe_debug_nvfp4_matmul_workspace_bytes(core, cols)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=codes.device)
    _check("moe_debug_nvfp4_matmul",
           lib().moe_debug_nvfp4_matmul(core, m, _ptr(codes), _ptr(scales), _ptr(wscale), N, K, _ptr(x),
                                        _ptr(x_scales), _ptr(inscale), cols, _ptr(out), _ptr(ws), ws.numel(),
                                        _stream()))
    return out


def workspace_views(ws, mode, T, k, E, H, I):
    """Typed views of a layer workspace: ids, weights, offsets, permutation, y_pairs, FFN part."""
    L = layer_workspace_layout(mode, T, k, E, H, I)
    P = T * k

    def view(name, n, dtype):
        nbytes = n * torch.empty(0, dtype=dtype).element_size()
        return ws[L[name]:L[name] + nbytes].view(dtype)

    return {
        "topk_ids": view("topk_ids", P, torch.int32).view(T, k),
        "topk_w": view("topk_w", P, torch.float32).view(T, k),
        "expert_offsets": view("expert_offsets", E + 1, torch.int32),
        "sorted_pairs": view("sorted_pairs", P, torch.int32),
        "pair_row": view("pair_row", P, torch.int32),
        "y_pairs": view("y_pairs", P * H, torch.float32).view(P, H),
        "ffn": ws[L["ffn"]:],
    }


def ffn_workspace_views(ws, mode, T, k, H, I):
    """Typed views of the expert workspace (the layout documented in the C header)."""
    P = T * k
    m = _mode(mode)
    o = 0
    out = {}

    def seg(name, nbytes, dtype, shape):
        nonlocal o
        n = nbytes // torch.empty(0, dtype=dtype).element_size()
        out[name] = ws[o:o + nbytes].view(dtype).view(*shape)
        o = (o + nbytes + 255) // 256 * 256
        del n

    n_plan = min(P, 1024) + P // 32
    if m == MOE_A16:
        seg("h", P * I * 2, torch.bfloat16, (P, I))   # (q4_g64_fp16 experts: fp16 bits)
        if T > 8:
            seg("plan", n_plan * 16, torch.int32, (n_plan, 4))
    elif m == MOE_A8:
        seg("x_codes", T * H, torch.uint8, (T, H))
        seg("x_scales", T * (H // 16) * 4, torch.float32, (T, H // 16))
        seg("h_codes", P * I, torch.uint8, (P, I))
        seg("h_scales", P * (I // 16) * 4, torch.float32, (P, I // 16))
        if T > 8:
            seg("plan", n_plan * 16, torch.int32, (n_plan, 4))
    else:
        seg("x_codes", P * 2 * (H // 2), torch.uint8, (P, 2, H // 2))
        seg("x_scales", P * 2 * (H // 16), torch.uint8, (P, 2, H // 16))
        seg("h_codes", P * (I // 2), torch.uint8, (P, I // 2))
        seg("h_scales", P * (I // 16), torch.uint8, (P, I // 16))
        seg("plan", n_plan * 16, torch.int32, (n_plan, 4))
    return out


def pack_experts(w_gu, w_dn, gu_inscale=None, dn_inscale=None):
    """NVFP4-pack fp32 expert weights on the GPU (each matrix under its own multiplier).

    w_gu float32 [E, 2I, H] (gate rows then up rows of each expert), w_dn float32
    [E, H, I].  Multipliers: f32(amax / 2688) per matrix (nvfp4_global_scale);
    codes and block scales: act_quant_nvfp4 with each row's matrix multiplier.
    """
    _need(w_gu, "w_gu", torch.float32)
    _need(w_dn, "w_dn", torch.float32)
    E, I2, H = w_gu.shape
    I = I2 // 2
    dev = w_gu.device
    g_gu = nvfp4_global_scale(w_gu.view(2 * E, I * H))
    rg = (torch.arange(E * 2 * I, device=dev, dtype=torch.int32) // I).contiguous()
    gu_codes, gu_scales = act_quant_nvfp4(w_gu.view(E * 2 * I, H), g_gu, rg)
    g_dn = nvfp4_global_scale(w_dn.view(E, H * I))
    rg = (torch.arange(E * H, device=dev, dtype=torch.int32) // H).contiguous()
    dn_codes, dn_scales = act_quant_nvfp4(w_dn.view(E * H, I), g_dn, rg)
    return Experts(gu_codes.view(E, 2 * I, H // 2), gu_scales.view(E, 2 * I, H // 16),
                   dn_codes.view(E, H, I // 2), dn_scales.view(E, H, I // 16),
                   g_gu.view(E, 2), g_dn, gu_inscale, dn_inscale)
