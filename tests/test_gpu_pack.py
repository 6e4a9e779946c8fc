"""moe_pack_fp4_scales on the GPU: the packed byte order the header states,
written out here as an index formula over the row-major array."""
import numpy as np
import pytest
import torch

import mixture_experts_amd as M

pytestmark = pytest.mark.gpu


def packed_reference(src: np.ndarray, rows: int, row_len: int, g: int) -> np.ndarray:
    """Byte ((b * (row_len/256) + s) * 32 + r) * R + j  <-  src[32b + r][s*R + j], R = 256/g."""
    R, runs = 256 // g, row_len // 256
    out = np.empty(rows * row_len // g, dtype=np.uint8)
    for row in range(rows):
        b, r = divmod(row, 32)
        for s in range(runs):
            at = ((b * runs + s) * 32 + r) * R
            out[at:at + R] = src[row, s * R:(s + 1) * R]
    return out


@pytest.mark.parametrize("recipe,g", [(M.RECIPE_MXFP4, 32), (M.RECIPE_NVFP4, 16)])
@pytest.mark.parametrize("rows,row_len", [(32, 256), (96, 768), (2 * 256, 1024)])
def test_pack_matches_the_stated_layout(recipe, g, rows, row_len):
    print(f"pack recipe={recipe} rows={rows} row_len={row_len}", flush=True)
    rng = np.random.default_rng(rows * 7 + row_len + g)
    src = rng.integers(0, 256, size=(rows, row_len // g), dtype=np.uint8)
    s_dev = torch.from_numpy(src).cuda()
    d_dev = torch.full((rows * row_len // g,), 0x5A, dtype=torch.uint8, device="cuda")
    M.moe_pack_fp4_scales(recipe, rows, row_len, s_dev, d_dev)
    torch.cuda.synchronize()
    assert np.array_equal(d_dev.cpu().numpy(), packed_reference(src, rows, row_len, g))
    assert np.array_equal(s_dev.cpu().numpy(), src)          # the input is not written


def test_pack_helper_keeps_expert_shape():
    """pack_fp4_scales on an [n][rows][row_len/G] expert stack packs all rows as one matrix."""
    rng = np.random.default_rng(5)
    src = rng.integers(0, 256, size=(3, 64, 512 // 32), dtype=np.uint8)
    out = M.pack_fp4_scales(M.RECIPE_MXFP4, torch.from_numpy(src).cuda())
    torch.cuda.synchronize()
    assert tuple(out.shape) == src.shape
    assert np.array_equal(out.cpu().numpy().reshape(-1), packed_reference(src.reshape(192, 16), 192, 512, 32))
