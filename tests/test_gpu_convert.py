"""moe_convert_mxfp4_to_fp8 on the GPU against the oracle's conversion (R14):
codes, block scales and the count of blocks not reproduced are bit-exact."""
import numpy as np
import pytest
import torch

import mixture_experts_amd as M
from oracle import moe_oracle as O
from workloads import configs as C
from workloads import generate as G

pytestmark = pytest.mark.gpu


def _convert(packed: np.ndarray, e8: np.ndarray):
    rows, half = packed.shape
    q = torch.from_numpy(packed).cuda()
    s = torch.from_numpy(e8).cuda()
    out = torch.full((rows, 2 * half), 0x5A, dtype=torch.uint8, device="cuda")
    sc = torch.full((rows // 128, 2 * half // 128), -1.0, dtype=torch.float32, device="cuda")
    bad = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    M.moe_convert_mxfp4_to_fp8(q, s, out, sc, bad)
    torch.cuda.synchronize()
    assert torch.equal(q.cpu(), torch.from_numpy(packed)) and torch.equal(s.cpu(), torch.from_numpy(e8))
    return out.cpu().numpy(), sc.cpu().numpy(), int(bad.item())


@pytest.mark.parametrize("rows,cols,seed", [(128, 128, 1), (256, 7168, 2), (2048, 1024, 3)])
def test_convert_generated_weights(rows, cols, seed):
    """MXFP4 weights from the workload encoder (N(0, 0.02) source values)."""
    print(f"convert rows={rows} cols={cols}", flush=True)
    w = torch.randn(rows, cols, generator=torch.Generator().manual_seed(seed)) * 0.02
    q, e8 = G.encode_mxfp4(w)
    got = _convert(q.numpy(), e8.numpy())
    want = O.convert_mxfp4_to_fp8(q.numpy(), e8.numpy())
    assert np.array_equal(got[0], want[0]), f"{(got[0] != want[0]).sum()} codes differ"
    assert np.array_equal(got[1], want[1])
    assert got[2] == want[2] == 0
    # lossless: the fp8 recipe's dequantisation gives back the MXFP4 values
    fp8 = O.dequant_expert(C.RECIPE_FP8_B128, {"w13": got[0], "w13_scale": got[1], "w2": got[0], "w2_scale": got[1]},
                           rows // 2, cols)[0]
    mx = O.dequant_expert(C.RECIPE_MXFP4, {"w13": q.numpy(), "w13_scale": e8.numpy(), "w2": q.numpy(),
                                           "w2_scale": e8.numpy()}, rows // 2, cols)[0]
    assert np.array_equal(fp8, mx)


def test_convert_wide_exponent_spread_rounds_and_counts():
    """Groups 9 to 40 binades below their block's largest: rounded like the oracle,
    every such block counted; all codes, signs of zero included, bit-exact."""
    rng = np.random.default_rng(9)
    rows, cols = 256, 512
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    e8 = (125 + rng.integers(0, 3, (rows, cols // 32))).astype(np.uint8)
    e8[3, 0] = 116
    e8[130, 9] = 100
    e8[200, 15] = 90
    e8[255, 4] = 1
    got = _convert(packed, e8)
    want = O.convert_mxfp4_to_fp8(packed, e8)
    assert np.array_equal(got[0], want[0]), f"{(got[0] != want[0]).sum()} codes differ"
    assert np.array_equal(got[1], want[1])
    assert got[2] == want[2] >= 3
