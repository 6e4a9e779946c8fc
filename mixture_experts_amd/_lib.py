"""ctypes binding of libmoe_mi355x.so (include/moe.h).  Argument marshalling only:
every step of the layer runs in the library's HIP kernels.  Tensors are torch
device tensors; the stream is torch's current HIP stream unless given."""
from __future__ import annotations

import contextlib
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")
# The same library with the GEMM kernels' 64-bit LDS-copy form forced on (tests only).
FLAT_LIB_PATH = os.path.join(_HERE, "libmoe_mi355x_flatcopy.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_LAUNCH = range(5)
RECIPE_F32, RECIPE_BF16, RECIPE_FP8_B128, RECIPE_MXFP4, RECIPE_NVFP4 = range(5)
SCORE_SIGMOID, SCORE_SQRTSOFTPLUS = range(2)

EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine",
           "moe_forward", "moe_forward_noalloc", "moe_forward_noalloc_scratch_bytes", "moe_rmsnorm",
           "moe_forward_residual", "moe_pack_fp4_scales", "moe_convert_mxfp4_to_fp8",
           "moe_status_string", "moe_profile_start", "moe_profile_stop", "moe_kernel_tag_name")
KERNEL_TAGS = ("gate_logits", "router", "perm_hist", "perm_scan", "perm_scatter", "gather", "tile_list",
               "ffn_gate_up", "ffn_down", "shared_gate_up", "shared_down_combine", "combine", "rmsnorm")


class MoeConfig(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("num_shared", ctypes.c_int32),
                ("shared_intermediate", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("score_func", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("recipe", ctypes.c_int32),
                ("swiglu_limit", ctypes.c_float)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p)]


class MoeError(RuntimeError):
    pass


_lib = None
_loaded = {}


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (there is no fallback).
    Without `path`: the library every call goes through (libmoe_mi355x.so unless
    `library()` has switched it)."""
    global _lib
    if path is None:
        if _lib is None:
            _lib = load(LIB_PATH)
        return _lib
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mixture_experts_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    cfgp = ctypes.POINTER(MoeConfig)
    wp = ctypes.POINTER(MoeWeights)
    lib.moe_workspace_bytes.argtypes = [cfgp]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_route.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_grouped_ffn.argtypes = [cfgp, vp, vp, vp, wp, vp, vp, sz, vp]
    lib.moe_combine.argtypes = [cfgp, vp, vp, vp, vp, wp, vp, vp, sz, vp]
    lib.moe_forward.argtypes = [cfgp, vp, vp, vp, wp, wp, vp, vp, vp, vp, sz, vp]
    lib.moe_forward_noalloc.argtypes = [cfgp, vp, vp, vp, wp, wp, vp, vp, vp, vp]
    lib.moe_forward_noalloc_scratch_bytes.argtypes = []
    lib.moe_forward_noalloc_scratch_bytes.restype = sz
    lib.moe_rmsnorm.argtypes = [cfgp, vp, vp, ctypes.c_float, vp, vp]
    lib.moe_forward_residual.argtypes = [cfgp, vp, vp, ctypes.c_float, vp, vp, wp, wp, vp, vp, vp, vp, sz, vp]
    lib.moe_pack_fp4_scales.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
    lib.moe_convert_mxfp4_to_fp8.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, vp, vp, vp, vp, vp]
    lib.moe_profile_start.argtypes = [ctypes.c_int32]
    lib.moe_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), ctypes.c_int32]
    lib.moe_kernel_tag_name.argtypes = [ctypes.c_int32]
    lib.moe_kernel_tag_name.restype = ctypes.c_char_p
    for name in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward", "moe_forward_noalloc",
                 "moe_rmsnorm",
                 "moe_forward_residual", "moe_pack_fp4_scales", "moe_convert_mxfp4_to_fp8", "moe_profile_start",
                 "moe_profile_stop"):
        getattr(lib, name).restype = i32
    _loaded[path] = lib
    return lib


@contextlib.contextmanager
def library(path: str):
    """Route every call of this module through another build of the library while
    the context is open (the tests' FLAT-copy build)."""
    global _lib
    saved = _lib
    _lib = load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def make_config(cfg) -> MoeConfig:
    """MoeConfig from any object with the layer attributes (e.g. workloads.configs.MoEConfig)."""
    return MoeConfig(int(cfg.num_tokens), int(cfg.hidden), int(cfg.num_experts), int(cfg.top_k),
                     int(cfg.intermediate), int(cfg.num_shared), int(cfg.shared_intermediate), int(cfg.n_group),
                     int(cfg.topk_group), int(cfg.score_func), int(bool(cfg.norm_topk_prob)),
                     float(cfg.routed_scaling_factor), int(cfg.recipe),
                     float(getattr(cfg, "swiglu_limit", 0.0)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status: int, what: str):
    if status != MOE_OK:
        msg = load().moe_status_string(status).decode()
        raise MoeError(f"{what}: {msg} (status {status})")


def make_weights(w13, w2, w13_scale=None, w2_scale=None) -> MoeWeights:
    """Pointers as they are (fp4 scales must already be in the packed layout)."""
    return MoeWeights(_ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale))


def moe_pack_fp4_scales(recipe, rows, row_len, src, dst, stream=None):
    _check(load().moe_pack_fp4_scales(int(recipe), int(rows), int(row_len), _ptr(src), _ptr(dst), _stream(stream)),
           "moe_pack_fp4_scales")


def pack_fp4_scales(recipe, scale, stream=None):
    """Row-major fp4 scales [n][rows][row_len/G] (uint8) -> a new tensor in the packed layout."""
    g = 32 if recipe == RECIPE_MXFP4 else 16
    out = scale.new_empty(scale.shape)
    moe_pack_fp4_scales(recipe, scale.numel() // scale.shape[-1], scale.shape[-1] * g, scale.contiguous(), out, stream)
    return out


def moe_convert_mxfp4_to_fp8(w_fp4, w_e8m0, w_fp8, w_fp8_scale, inexact_blocks=None, stream=None):
    """MXFP4 [rows][row_len/2] + row-major E8M0 [rows][row_len/32] -> e4m3fn codes
    [rows][row_len] + fp32 scales [rows/128][row_len/128] (include/moe.h)."""
    rows = w_fp4.numel() // w_fp4.shape[-1]
    _check(load().moe_convert_mxfp4_to_fp8(int(rows), int(w_fp4.shape[-1] * 2), _ptr(w_fp4), _ptr(w_e8m0),
                                           _ptr(w_fp8), _ptr(w_fp8_scale), _ptr(inexact_blocks), _stream(stream)),
           "moe_convert_mxfp4_to_fp8")


def make_expert_weights(recipe, w13, w2, w13_scale=None, w2_scale=None, stream=None) -> MoeWeights:
    """Routed-expert weights as the layer call reads them.  MXFP4 / NVFP4 scales
    (row-major, as quantised) are packed into new device tensors once, here; the
    returned struct keeps them alive."""
    if recipe in (RECIPE_MXFP4, RECIPE_NVFP4):
        w13_scale = pack_fp4_scales(recipe, w13_scale, stream)
        w2_scale = pack_fp4_scales(recipe, w2_scale, stream)
    wts = make_weights(w13, w2, w13_scale, w2_scale)
    wts._keep = (w13, w2, w13_scale, w2_scale)
    return wts


def moe_workspace_bytes(cfg: MoeConfig) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(cfg)))


def moe_route(cfg, x, gate_w, bias, topk_idx, topk_w, ws, stream=None):
    _check(load().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(gate_w), _ptr(bias), _ptr(topk_idx), _ptr(topk_w),
                            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_route")


def moe_permute(cfg, topk_idx, x, expert_offsets, sorted_pair, pair_pos, x_perm, x_perm_scale, ws, stream=None):
    _check(load().moe_permute(ctypes.byref(cfg), _ptr(topk_idx), _ptr(x), _ptr(expert_offsets), _ptr(sorted_pair),
                              _ptr(pair_pos), _ptr(x_perm), _ptr(x_perm_scale), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "moe_permute")


def moe_grouped_ffn(cfg, expert_offsets, x_perm, x_perm_scale, experts: MoeWeights, y_perm, ws, stream=None):
    _check(load().moe_grouped_ffn(ctypes.byref(cfg), _ptr(expert_offsets), _ptr(x_perm), _ptr(x_perm_scale),
                                  ctypes.byref(experts), _ptr(y_perm), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "moe_grouped_ffn")


def moe_combine(cfg, y_perm, pair_pos, topk_w, x, shared: MoeWeights | None, out, ws, stream=None):
    _check(load().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(pair_pos), _ptr(topk_w), _ptr(x),
                              ctypes.byref(shared) if shared is not None else None, _ptr(out), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "moe_combine")


def moe_forward(cfg, x, gate_w, bias, experts: MoeWeights, shared: MoeWeights | None, out, topk_idx_out, topk_w_out,
                ws, stream=None):
    _check(load().moe_forward(ctypes.byref(cfg), _ptr(x), _ptr(gate_w), _ptr(bias), ctypes.byref(experts),
                              ctypes.byref(shared) if shared is not None else None, _ptr(out), _ptr(topk_idx_out),
                              _ptr(topk_w_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_forward")


def moe_forward_noalloc(cfg, x, gate_w, bias, experts: MoeWeights, shared: MoeWeights | None, out, topk_idx_out,
                        topk_w_out, stream=None):
    """moe_forward with the library's static scratch instead of a workspace (include/moe.h)."""
    _check(load().moe_forward_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(gate_w), _ptr(bias), ctypes.byref(experts),
                                      ctypes.byref(shared) if shared is not None else None, _ptr(out),
                                      _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream)), "moe_forward_noalloc")


def moe_forward_noalloc_scratch_bytes() -> int:
    return int(load().moe_forward_noalloc_scratch_bytes())


def moe_rmsnorm(cfg, resid, norm_w, eps: float, x, stream=None):
    _check(load().moe_rmsnorm(ctypes.byref(cfg), _ptr(resid), _ptr(norm_w), float(eps), _ptr(x), _stream(stream)),
           "moe_rmsnorm")


def moe_forward_residual(cfg, resid, norm_w, eps: float, gate_w, bias, experts: MoeWeights,
                         shared: MoeWeights | None, out, topk_idx_out, topk_w_out, ws, stream=None):
    _check(load().moe_forward_residual(ctypes.byref(cfg), _ptr(resid), _ptr(norm_w), float(eps), _ptr(gate_w),
                                       _ptr(bias), ctypes.byref(experts),
                                       ctypes.byref(shared) if shared is not None else None, _ptr(out),
                                       _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)), "moe_forward_residual")


def moe_profile_start(max_launches: int = 4096):
    _check(load().moe_profile_start(int(max_launches)), "moe_profile_start")


def moe_profile_stop() -> dict:
    """{kernel tag name: (summed ms, launches)} for the launches recorded since start."""
    n = len(KERNEL_TAGS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(load().moe_profile_stop(ms, cnt, n), "moe_profile_stop")
    return {KERNEL_TAGS[i]: (ms[i], int(cnt[i])) for i in range(n)}
