"""The C-ABI library: it loads, exports every symbol include/moe.h declares, and
rejects bad arguments on the host before touching the GPU.  CPU only."""
import ctypes
import os
import re

import pytest

import mixture_experts_amd as M
from workloads import configs as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(M.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    lib = M.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_config_struct_matches_header_layout():
    # 12 int32 + 2 float, no padding
    assert ctypes.sizeof(M.MoeConfig) == 14 * 4
    assert ctypes.sizeof(M.MoeWeights) == 4 * ctypes.sizeof(ctypes.c_void_p)


def test_status_strings():
    lib = M.load()
    assert lib.moe_status_string(0) == b"ok"
    assert b"workspace" in lib.moe_status_string(3)


@pytest.mark.parametrize("cfg", C.FULL_CONFIGS + C.MINI_CONFIGS, ids=lambda c: c.name)
def test_workspace_sizes_are_positive_for_every_workload(cfg):
    n = M.moe_workspace_bytes(M.make_config(cfg))
    P, H = cfg.pairs, cfg.hidden
    assert n >= P * H  # at least the permuted activations
    assert n < 8 << 30


BAD = [
    dict(n_group=3),                       # E % n_group != 0 for E=16
    dict(n_group=4, topk_group=5),         # topk_group > n_group
    dict(n_group=16, topk_group=1),        # one expert per group
    dict(n_group=4, topk_group=1, top_k=5),  # kept experts < k
    dict(top_k=17),
    dict(top_k=0),
    dict(num_experts=2000, top_k=4),
    dict(score_func=7),
    dict(recipe=9),
    dict(swiglu_limit=-1.0),
    dict(swiglu_limit=float("nan")),
    dict(swiglu_limit=float("inf")),
]


@pytest.mark.parametrize("bad", BAD, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_invalid_configs_are_rejected_without_launch(bad):
    cfg = M.make_config(C.TINY_F32.replace(**bad))
    assert M.moe_workspace_bytes(cfg) == 0
    lib = M.load()
    st = lib.moe_route(ctypes.byref(cfg), None, None, None, None, None, None, 0, None)
    assert st == 1  # MOE_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("base,change", [
    (C.DECODE_BF16, dict(hidden=7100)),
    (C.MINI_MXFP4, dict(hidden=384)),          # fp4 recipes: multiples of 256
    (C.MINI_NVFP4, dict(intermediate=384)),
], ids=["bf16-hidden-7100", "mxfp4-hidden-384", "nvfp4-intermediate-384"])
def test_unsupported_shapes_report_unsupported(base, change):
    cfg = M.make_config(base.replace(**change))
    assert M.moe_workspace_bytes(cfg) == 0
    st = M.load().moe_forward(ctypes.byref(cfg), None, None, None, None, None, None, None, None, None, 0, None)
    assert st == 2  # MOE_ERR_UNSUPPORTED


def test_null_pointers_and_small_workspace_are_rejected():
    lib = M.load()
    cfg = M.make_config(C.TINY_F32)
    ws = ctypes.c_void_p(1 << 20)          # never dereferenced: validation fails first
    st = lib.moe_route(ctypes.byref(cfg), None, None, None, None, None, ws, M.moe_workspace_bytes(cfg), None)
    assert st == 1
    fake = ctypes.c_void_p(4096)
    st = lib.moe_route(ctypes.byref(cfg), fake, fake, fake, fake, fake, ws, 16, None)
    assert st == 3  # MOE_ERR_WORKSPACE_TOO_SMALL
    misaligned = ctypes.c_void_p((1 << 20) + 8)
    st = lib.moe_route(ctypes.byref(cfg), fake, fake, fake, fake, fake, misaligned, 1 << 40, None)
    assert st == 1


def test_zero_tokens_is_a_no_op():
    lib = M.load()
    cfg = M.make_config(C.TINY_F32.replace(num_tokens=0))
    assert lib.moe_forward(ctypes.byref(cfg), None, None, None, None, None, None, None, None, None, 0, None) == 0


@pytest.mark.parametrize("recipe,rows,row_len,src,dst,want", [
    (M.RECIPE_BF16, 32, 256, 1 << 20, 1 << 24, 1),           # only the fp4 recipes have packed scales
    (M.RECIPE_FP8_B128, 32, 256, 1 << 20, 1 << 24, 1),
    (M.RECIPE_MXFP4, -32, 256, 1 << 20, 1 << 24, 1),
    (M.RECIPE_MXFP4, 32, 0, 1 << 20, 1 << 24, 1),
    (M.RECIPE_MXFP4, 48, 256, 1 << 20, 1 << 24, 2),          # rows not a multiple of 32
    (M.RECIPE_NVFP4, 32, 384, 1 << 20, 1 << 24, 2),          # row length not a multiple of 256
    (M.RECIPE_MXFP4, 32, 256, None, 1 << 24, 1),
    (M.RECIPE_NVFP4, 32, 256, (1 << 20) + 8, 1 << 24, 1),    # misaligned
    (M.RECIPE_MXFP4, 64, 1024, 1 << 20, (1 << 20) + 1024, 1),  # 1 KiB apart: the 2 KiB arrays overlap
    (M.RECIPE_MXFP4, 0, 256, None, None, 0),                 # no rows: a no-op
])
def test_pack_fp4_scales_argument_checks(recipe, rows, row_len, src, dst, want):
    """Rejected before anything is enqueued (the pointers are never dereferenced)."""
    lib = M.load()
    p = lambda a: None if a is None else ctypes.c_void_p(a)
    assert lib.moe_pack_fp4_scales(recipe, rows, row_len, p(src), p(dst), None) == want


@pytest.mark.parametrize("rows,row_len,ptrs,want", [
    (-128, 256, (1 << 20, 1 << 21, 1 << 22, 1 << 23, None), 1),
    (128, 0, (1 << 20, 1 << 21, 1 << 22, 1 << 23, None), 1),
    (96, 256, (1 << 20, 1 << 21, 1 << 22, 1 << 23, None), 2),     # rows not a multiple of 128
    (128, 192, (1 << 20, 1 << 21, 1 << 22, 1 << 23, None), 2),    # row length not a multiple of 128
    (128, 256, (None, 1 << 21, 1 << 22, 1 << 23, None), 1),
    (128, 256, (1 << 20, 1 << 21, None, 1 << 23, None), 1),
    (128, 256, (1 << 20, (1 << 21) + 2, 1 << 22, 1 << 23, None), 1),   # misaligned scales
    (128, 256, (1 << 20, 1 << 21, 1 << 22, 1 << 23, (1 << 24) + 2), 1),   # misaligned counter
    (0, 256, (None, None, None, None, None), 0),                    # no rows: a no-op
])
def test_convert_mxfp4_to_fp8_argument_checks(rows, row_len, ptrs, want):
    """Rejected before anything is enqueued (the pointers are never dereferenced)."""
    lib = M.load()
    p = lambda a: None if a is None else ctypes.c_void_p(a)
    assert lib.moe_convert_mxfp4_to_fp8(rows, row_len, *[p(a) for a in ptrs], None) == want
