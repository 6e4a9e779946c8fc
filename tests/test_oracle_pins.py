"""Pins for the CPU oracle: checks against what the pages and the mathematics fix,
never against the oracle's own formulas retyped.  CPU only."""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import configs as C
from workloads import generate as G

HERE = os.path.dirname(os.path.abspath(__file__))
F32 = np.float32


# ------------------------------------------------------------------ helpers
def fp32_nearest(fr: Fraction) -> np.float32:
    """The fp32 nearest to an exact rational (ties to even), by exact comparison of neighbours."""
    r = np.float32(float(fr))
    cands = [np.nextafter(r, F32(-np.inf)), r, np.nextafter(r, F32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, dtype=F32).view(np.uint32)) & 1))
    return F32(best)


def rand_small_cfg(**kw):
    base = dict(name="pin", num_tokens=40, hidden=64, num_experts=16, top_k=4, intermediate=32,
                num_shared=1, shared_intermediate=16, recipe=C.RECIPE_F32)
    base.update(kw)
    return C.MoEConfig(**base)


def brute_select(key_row, n_group, topk_group, k):
    """Selection by full sorts of Python tuples (page: group top-2 sums, keep groups, top-k)."""
    E = len(key_row)
    keys = [float(v) for v in key_row]
    if n_group > 1:
        gs = E // n_group
        gscores = []
        for g in range(n_group):
            members = sorted(keys[g * gs:(g + 1) * gs], reverse=True)
            gscores.append((-float(F32(members[0]) + F32(members[1])), g))
        kept_groups = {g for _, g in sorted(gscores)[:topk_group]}
        cand = [e for e in range(E) if e // gs in kept_groups]
    else:
        cand = list(range(E))
    return [e for _, e in sorted((-keys[e], e) for e in cand)[:k]]


# ------------------------------------------------------------------ score functions
def test_score_closed_forms():
    z = np.array([0.0], dtype=F32)
    assert O.score(z, O.SCORE_SIGMOID)[0] == F32(0.5)
    # sqrt(softplus(0)) = sqrt(ln 2) = 0.83255461115769775...
    assert O.score(z, O.SCORE_SQRTSOFTPLUS)[0] == F32(0.8325546111576977)
    # large z: softplus(z) -> z, so sqrtsoftplus(z) -> sqrt(z); sigmoid -> 1
    big = np.array([60.0, 100.0], dtype=F32)
    assert np.array_equal(O.score(big, O.SCORE_SQRTSOFTPLUS), np.sqrt(big.astype(np.float64)).astype(F32))
    assert np.all(O.score(big, O.SCORE_SIGMOID) == F32(1.0))
    # very negative: sigmoid(z) ~ e^z, sqrtsoftplus(z) ~ e^(z/2)
    neg = np.array([-40.0], dtype=F32)
    assert O.score(neg, O.SCORE_SIGMOID)[0] == F32(math.exp(-40.0))
    assert O.score(neg, O.SCORE_SQRTSOFTPLUS)[0] == F32(math.exp(-20.0))


def test_score_monotone():
    z = np.sort(np.random.default_rng(1).standard_normal(5000).astype(F32) * 8)
    for f in (O.SCORE_SIGMOID, O.SCORE_SQRTSOFTPLUS):
        s = O.score(z, f)
        assert np.all(np.diff(s.astype(np.float64)) >= 0)


def test_score_correctly_rounded_decimal():
    getcontext().prec = 60
    rng = np.random.default_rng(2)
    z = (rng.standard_normal(400) * 3).astype(F32)
    sig = O.score(z, O.SCORE_SIGMOID)
    ssp = O.score(z, O.SCORE_SQRTSOFTPLUS)
    for zi, a, b in zip(z, sig, ssp):
        d = Decimal(float(zi))
        exact_sig = 1 / (1 + (-d).exp())
        exact_ssp = (1 + d.exp()).ln().sqrt()
        for got, exact in ((a, exact_sig), (b, exact_ssp)):
            fr = Fraction(exact)
            assert fp32_nearest(fr) == got, (zi, got)


# ------------------------------------------------------------------ logits
def test_logits_are_correctly_rounded_dot_products():
    rng = np.random.default_rng(3)
    T, E, H = 12, 10, 96
    x = rng.standard_normal((T, H)).astype(F32)
    # bf16-valued x as in the bf16 recipes: keep the top 16 bits
    xb = (x.view(np.uint32) & 0xFFFF0000).view(F32)
    w = (rng.standard_normal((E, H)) * 0.1).astype(F32)
    for xx in (x, xb):
        got = O.gate_logits(xx.astype(np.float64), w.astype(np.float64))
        for t in range(T):
            for e in range(E):
                exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xx[t], w[e]))
                assert got[t, e] == fp32_nearest(exact)


# ------------------------------------------------------------------ selection
@pytest.mark.parametrize("E,n_group,topk_group,k", [(16, 1, 1, 4), (32, 4, 2, 6), (32, 8, 4, 8),
                                                    (24, 3, 1, 5), (64, 8, 3, 8)])
def test_topk_matches_bruteforce(E, n_group, topk_group, k):
    cfg = rand_small_cfg(num_experts=E, top_k=k, n_group=n_group, topk_group=topk_group)
    rng = np.random.default_rng(E + k)
    T, H = 50, 64
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((E, H)) / 8
    b = (rng.uniform(-0.1, 0.1, E)).astype(F32)
    r = O.route(cfg, x, wg, b)
    for t in range(T):
        assert list(r["idx"][t]) == brute_select(r["key"][t], n_group, topk_group, k)


def test_group_step_is_identity_when_one_group_or_all_groups_kept():
    rng = np.random.default_rng(5)
    T, H, E, k = 60, 64, 32, 6
    x = rng.standard_normal((T, H)); wg = rng.standard_normal((E, H)) / 8
    b = rng.uniform(-0.1, 0.1, E).astype(F32)
    plain = rand_small_cfg(num_experts=E, top_k=k)
    ref = O.route(plain, x, wg, b)["idx"]
    # plain top-k written as a full argsort of (-key, index)
    key = O.route(plain, x, wg, b)["key"]
    for t in range(T):
        assert list(ref[t]) == [e for _, e in sorted((-float(v), e) for e, v in enumerate(key[t]))][:k]
    allkept = rand_small_cfg(num_experts=E, top_k=k, n_group=4, topk_group=4)
    assert np.array_equal(O.route(allkept, x, wg, b)["idx"], ref)


def test_exact_ties_go_to_lowest_index():
    T, H, E, k = 8, 32, 16, 4
    rng = np.random.default_rng(6)
    x = rng.standard_normal((T, H))
    row = rng.standard_normal(H) / 8
    wg = np.tile(row, (E, 1))                       # every expert has the same gate row
    b = np.zeros(E, dtype=F32)
    r = O.route(rand_small_cfg(num_experts=E, top_k=k), x, wg, b)
    assert np.all(r["idx"] == np.arange(k))
    rg = O.route(rand_small_cfg(num_experts=E, top_k=k, n_group=4, topk_group=2), x, wg, b)
    assert np.all(rg["idx"] == np.arange(k))         # groups 0, 1 kept; experts 0..3
    # twins at the boundary: experts 9 and 3 have identical gate rows and bias;
    # whenever only one of them makes the cut it must be 3
    T2 = 64
    x2 = rng.standard_normal((T2, H))
    wg2 = rng.standard_normal((E, H)) / 8
    wg2[9] = wg2[3]
    b2 = np.full(E, -5.0, dtype=F32); b2[[1, 3, 9, 12]] = 5.0; b2[5] = 6.0
    r2 = O.route(rand_small_cfg(num_experts=E, top_k=4), x2, wg2, b2)
    only_one = 0
    for t in range(T2):
        sel = set(r2["idx"][t].tolist())
        assert 5 in sel
        assert (9 not in sel) or (3 in sel)
        only_one += (3 in sel) and (9 not in sel)
    assert only_one > 0


# ------------------------------------------------------------------ weights
@pytest.mark.parametrize("func,scale", [(O.SCORE_SIGMOID, 2.827), (O.SCORE_SQRTSOFTPLUS, 2.5)])
def test_weights_sum_to_scale_and_positive(func, scale):
    rng = np.random.default_rng(7)
    cfg = rand_small_cfg(num_experts=32, top_k=8, score_func=func, routed_scaling_factor=scale)
    x = rng.standard_normal((100, 64)); wg = rng.standard_normal((32, 64)) / 8
    b = rng.normal(0, 0.01, 32).astype(F32)
    w = O.route(cfg, x, wg, b)["w"].astype(np.float64)
    assert np.all(w > 0)
    assert np.all(np.abs(w.sum(axis=1) - scale) <= 8 * 2.0 ** -23 * scale)


def test_forcing_bias_selects_and_weights_use_unbiased_scores():
    rng = np.random.default_rng(8)
    E, k, H, T = 16, 4, 64, 30
    x = rng.standard_normal((T, H)); wg = rng.standard_normal((E, H)) / 8
    b = np.zeros(E, dtype=F32); b[:k] = 10.0
    cfg = rand_small_cfg(num_experts=E, top_k=k, routed_scaling_factor=2.827)
    r = O.route(cfg, x, wg, b)
    for t in range(T):
        assert sorted(r["idx"][t].tolist()) == list(range(k))
        # weights proportional to sigma(logit) of the chosen experts, not to sigma + 10
        z = np.array([float(np.dot(x[t], wg[e])) for e in r["idx"][t]])
        sig = 1 / (1 + np.exp(-z))
        np.testing.assert_allclose(r["w"][t], sig / sig.sum() * 2.827, rtol=2e-6)


# ------------------------------------------------------------------ permutation
def test_permutation_invariants_and_round_trip():
    rng = np.random.default_rng(9)
    T, k, E = 257, 6, 40
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    for t in range(50):                                # a popular expert (no token picks it twice)
        if 3 not in idx[t]:
            idx[t, 0] = 3
    p = O.permute(idx, E)
    assert p["counts"].sum() == T * k
    assert p["offsets"][0] == 0 and np.array_equal(np.diff(p["offsets"]), p["counts"])
    assert np.array_equal(np.sort(p["sorted_pair"]), np.arange(T * k))          # bijection
    flat = idx.reshape(-1)
    for e in range(E):
        blk = p["sorted_pair"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(flat[blk] == e)                                           # contiguous block
        assert np.all(np.diff(blk // k) > 0)                                   # ascending tokens
    rows = np.arange(T * k)[p["sorted_pair"]]          # permute...
    assert np.array_equal(rows[p["pair_pos"]], np.arange(T * k))               # ...and back
    # un-permute of data rows restores original order exactly
    data = rng.standard_normal((T * k, 3))
    assert np.array_equal(data[p["sorted_pair"]][p["pair_pos"]], data)


# ------------------------------------------------------------------ FFN
def _loops_mlp(x, w13, w2):
    I = len(w13) // 2
    out = []
    for row in x:
        h = []
        for i in range(I):
            g = sum(a * b for a, b in zip(row, w13[i]))
            u = sum(a * b for a, b in zip(row, w13[I + i]))
            h.append(g / (1 + math.exp(-g)) * u)
        out.append([sum(a * b for a, b in zip(h, w2[n])) for n in range(len(w2))])
    return np.array(out)


def test_expert_mlp_matches_scalar_loops():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((3, 8)); w13 = rng.standard_normal((8, 8)); w2 = rng.standard_normal((8, 4))
    np.testing.assert_allclose(O.expert_mlp(x, w13, w2), _loops_mlp(x, w13, w2), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ method variants
def test_unnormalised_weights_are_the_scaled_scores_of_the_picks():
    """norm_topk_prob = false (walk-through 3.3 normalises only when the flag is set):
    the weights keep the ratios of the normalised ones and sum to scale * (sum of
    the picked scores), each in (0, scale) for sigmoid scores."""
    rng = np.random.default_rng(11)
    cfg = rand_small_cfg(num_experts=32, top_k=8, routed_scaling_factor=2.827)
    x = rng.standard_normal((60, 64)); wg = rng.standard_normal((32, 64)) / 8
    b = rng.normal(0, 0.01, 32).astype(F32)
    rn = O.route(cfg, x, wg, b)
    ru = O.route(cfg.replace(norm_topk_prob=False), x, wg, b)
    assert np.array_equal(rn["idx"], ru["idx"])                      # selection does not depend on it
    wn, wu = rn["w"].astype(np.float64), ru["w"].astype(np.float64)
    assert np.all((wu > 0) & (wu < 2.827))
    ssum = wu.sum(axis=1, keepdims=True) / 2.827                      # sum of the picked scores
    np.testing.assert_allclose(wn * ssum, wu, rtol=1e-6)
    assert np.all(np.abs(ssum - 1.0) > 1e-3)                          # the two variants differ


def test_swiglu_limit_zero_or_huge_is_plain_swiglu():
    rng = np.random.default_rng(12)
    g, u = rng.standard_normal((2, 500)) * 3
    plain = O.silu(g) * u
    assert np.array_equal(O.swiglu(g, u, 0.0), plain)
    assert np.array_equal(O.swiglu(g, u, 1e30), plain)


def test_swiglu_limit_saturates_as_read():
    """The reading of the optional truncation: gate clamped from above only, up
    clamped on both sides, SiLU applied after."""
    L = 1.0
    silu_L = 1.0 / (1.0 + math.exp(-1.0))                             # SiLU(1)
    u = np.array([-3.0, -0.5, 0.0, 0.7, 5.0])
    # gate above the limit: SiLU(L) * clamp(u)
    np.testing.assert_allclose(O.swiglu(np.full(5, 7.0), u, L), silu_L * np.array([-1.0, -0.5, 0.0, 0.7, 1.0]),
                               rtol=1e-15)
    # gate far below -L is not raised to -L: SiLU(-10) * u, not SiLU(-1) * u
    silu_m10 = -10.0 / (1.0 + math.exp(10.0))
    np.testing.assert_allclose(O.swiglu(np.full(5, -10.0), u, L), silu_m10 * np.clip(u, -1, 1), rtol=1e-12)
    # inside the box nothing changes
    gi = np.array([-0.9, -0.2, 0.3, 0.99, 1.0])
    ui = np.array([0.5, -1.0, 1.0, -0.3, 0.2])
    np.testing.assert_allclose(O.swiglu(gi, ui, L), gi / (1 + np.exp(-gi)) * ui, rtol=1e-15)
    # bounded output: |h| <= L * max(SiLU(L), -min SiLU) for any input
    rng = np.random.default_rng(13)
    g, uu = rng.standard_normal((2, 10000)) * 20
    assert np.all(np.abs(O.swiglu(g, uu, L)) <= L * max(silu_L, 0.27846454) + 1e-12)


def test_swiglu_limit_in_the_expert_mlp_matches_scalar_loops():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((3, 8)); w13 = rng.standard_normal((8, 8)); w2 = rng.standard_normal((8, 4))
    L = 0.8
    I = 4
    want = []
    for row in x:
        h = []
        for i in range(I):
            g = sum(a * b for a, b in zip(row, w13[i]))
            u = sum(a * b for a, b in zip(row, w13[I + i]))
            if g > L:
                g = L
            if u > L:
                u = L
            elif u < -L:
                u = -L
            h.append(g / (1 + math.exp(-g)) * u)
        want.append([sum(a * b for a, b in zip(h, w2[n])) for n in range(len(w2))])
    np.testing.assert_allclose(O.expert_mlp(x, w13, w2, limit=L), np.array(want), rtol=1e-12, atol=1e-12)


def _f32_raw(w13, w2):
    return lambda e: {"w13": w13[e], "w2": w2[e]}


def test_single_expert_layer_is_textbook_swiglu():
    rng = np.random.default_rng(11)
    T, H, I = 5, 8, 6
    cfg = rand_small_cfg(num_tokens=T, hidden=H, num_experts=1, top_k=1, intermediate=I,
                         shared_intermediate=4, routed_scaling_factor=1.0)
    x = rng.standard_normal((T, H)); wg = rng.standard_normal((1, H))
    w13 = rng.standard_normal((1, 2 * I, H)).astype(F32); w2 = rng.standard_normal((1, H, I)).astype(F32)
    s13 = rng.standard_normal((1, 8, H)); s2 = rng.standard_normal((1, H, 4))
    r = O.moe_forward(cfg, x, wg, np.zeros(1, F32), _f32_raw(w13, w2), s13, s2)
    want = _loops_mlp(x, w13[0].astype(np.float64), w2[0].astype(np.float64)) + _loops_mlp(x, s13[0], s2[0])
    np.testing.assert_allclose(r["out"], want, rtol=1e-12, atol=1e-12)


def test_sparse_layer_equals_dense_bruteforce():
    rng = np.random.default_rng(12)
    T, H, E, k, I = 7, 16, 8, 3, 8
    cfg = rand_small_cfg(num_tokens=T, hidden=H, num_experts=E, top_k=k, intermediate=I,
                         num_shared=2, shared_intermediate=4, n_group=2, topk_group=1,
                         routed_scaling_factor=2.827)
    x = rng.standard_normal((T, H)); wg = rng.standard_normal((E, H)) / 4
    b = rng.uniform(-0.1, 0.1, E).astype(F32)
    w13 = rng.standard_normal((E, 2 * I, H)).astype(F32); w2 = rng.standard_normal((E, H, I)).astype(F32)
    s13 = rng.standard_normal((2, 8, H)); s2 = rng.standard_normal((2, H, 4))
    r = O.moe_forward(cfg, x, wg, b, _f32_raw(w13, w2), s13, s2)
    dense_w = np.zeros((T, E))
    np.put_along_axis(dense_w, r["routing"]["idx"].astype(np.int64), r["routing"]["w"].astype(np.float64), 1)
    want = np.zeros((T, H))
    for e in range(E):                                  # every expert on every token
        want += dense_w[:, e:e + 1] * _loops_mlp(x, w13[e].astype(np.float64), w2[e].astype(np.float64))
    for s in range(2):
        want += _loops_mlp(x, s13[s], s2[s])
    np.testing.assert_allclose(r["out"], want, rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------------ number formats
def test_e2m1_grid_and_e8m0():
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    v = O.decode_e2m1_packed(packed[None])[0]
    assert list(v[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(v[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    e8 = O.decode_e8m0(np.array([0, 126, 127, 128, 254, 255], dtype=np.uint8))
    assert list(e8[:5]) == [2.0 ** -127, 0.5, 1.0, 2.0, 2.0 ** 127] and math.isnan(e8[5])


def test_e4m3_decode_matches_torch_and_max_is_448():
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    o = O.decode_e4m3(codes)
    assert np.array_equal(np.isnan(t), np.isnan(o)) and np.array_equal(t[~np.isnan(t)], o[~np.isnan(o)])
    assert np.nanmax(o) == 448.0 and np.isnan(o[0x7F]) and np.isnan(o[0xFF])


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(13)
    mids = O._E4M3_MID
    v = np.concatenate([rng.standard_normal(200000) * 64, rng.standard_normal(20000) * 1e-2,
                        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [0.0, -0.0, 1e-12, -1e-12, 448.0, -448.0]]).astype(F32)
    v = np.clip(v, -448, 448)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_e4m3(v), want)


def test_every_e2m1_value_is_exact_in_e4m3():
    """FP4 -> FP8 conversion (e2m1fn -> e4m3fn) is lossless; checked through the oracle's codecs."""
    page = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))
    assert page["e2m1_to_e4m3_lossless"]["value"] is True
    e2m1 = O.E2M1_TABLE
    for scale_exp in range(-6, 4):                     # with any power-of-two block scale in range
        v = e2m1 * 2.0 ** scale_exp
        back = O.decode_e4m3(O.encode_e4m3(v))
        assert np.array_equal(back, v)


def test_mx_exponent_is_least_that_fits():
    rng = np.random.default_rng(14)
    a = np.abs(rng.standard_normal(20000)) * 10.0 ** rng.uniform(-6, 6, 20000)
    a = np.concatenate([a, 448.0 * 2.0 ** np.arange(-20, 20)])       # exact powers on the edge
    e = O.mx_exponent(a, 448.0)
    assert np.all(a <= 448.0 * np.ldexp(1.0, e))
    assert np.all(a > 448.0 * np.ldexp(1.0, e - 1))


def test_activation_quantisers_bound_and_round_trip():
    rng = np.random.default_rng(15)
    v = (rng.standard_normal((9, 256)) * 3).astype(F32)
    v[2, :128] = 0.0                                   # an all-zero block
    q, s = O.quant_fp8_b128(v)
    assert s[2, 0] == 1.0 and np.all(q[2, :128] & 0x7F == 0)
    d = O.dequant_fp8_b128(q, s)
    assert np.all(np.abs(d - v) <= np.abs(v) * 2.0 ** -4 + s.repeat(128, 1) * 2.0 ** -10)
    assert np.all(np.abs(O.decode_e4m3(q)) <= 448.0)
    # quantising the dequantised values again gives the same codes (Q(D(q)) = q)
    q2, s2 = O.quant_fp8_b128(d.astype(F32))
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    qm, em = O.quant_mxfp8(v)
    dm = O.dequant_mxfp8(qm, em)
    assert np.all(np.abs(dm - v) <= np.abs(v) * 2.0 ** -4 + O.decode_e8m0(em).repeat(32, 1) * 2.0 ** -9)
    # dequantised values are exactly representable: quantising them again loses nothing
    # (codes may differ: a block whose amax rounded down to 224*2^e re-quantises with e - 1)
    q3, e3 = O.quant_mxfp8(dm.astype(F32))
    assert np.array_equal(O.dequant_mxfp8(q3, e3), dm)


# ------------------------------------------------------------------ page constants
def test_page_constants_and_mxfp4_byte_accounting():
    page = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))
    assert C.DECODE_BF16.routed_scaling_factor == page["routed_scaling_factor_v3"]["value"]
    assert C.SKEWED_FP8.routed_scaling_factor == page["route_scale_v4"]["value"]
    v3, v4, k3 = page["v3_experts"], page["v4_experts"], page["k3_experts"]
    assert (C.DECODE_BF16.num_experts, C.DECODE_BF16.top_k, C.DECODE_BF16.num_shared,
            C.DECODE_BF16.hidden) == (v3["routed"], v3["top_k"], v3["shared"], v3["hidden"])
    assert (C.SKEWED_FP8.num_experts, C.SKEWED_FP8.top_k, C.SKEWED_FP8.num_shared) == \
        (v4["routed"], v4["top_k"], v4["shared"])
    assert (C.FINEGRAINED_MXFP4.num_experts, C.FINEGRAINED_MXFP4.top_k, C.FINEGRAINED_MXFP4.num_shared) == \
        (k3["routed"], k3["top_k"], k3["shared"])
    st = page["mxfp4_storage"]
    lower = st["params"] * st["bits"] / 8 / 1e12
    assert abs(lower - st["lower_bound_TB"]) < 0.005
    with_scales = st["params"] * O.mxfp4_bytes_per_param() / 1e12
    assert st["lower_bound_TB"] < with_scales < st["stored_TB"]
    assert st["params"] * 2 / 1e12 >= st["unquantised_16bit_TB_at_least"]


# ------------------------------------------------------------------ residual form (RMSNorm)
def test_encode_bf16_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(15)
    v = np.concatenate([rng.standard_normal(5000).astype(F32) * 10.0 ** rng.integers(-6, 6, 5000),
                        # exact ties between two bf16 neighbours: low 16 bits 0x8000
                        (rng.integers(0x3F000000, 0x40800000, 200).astype(np.uint32) & 0xFFFF0000 | 0x8000)
                        .view(F32)]).astype(F32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.encode_bf16(v), want)


@pytest.mark.parametrize("recipe", [O.RECIPE_F32, O.RECIPE_BF16])
def test_rms_norm_closed_forms(recipe):
    H = 256
    # a constant row c: mean square c^2, so with eps = 0 and unit weight every entry is sign(c)
    h = np.array([[0.75] * H, [-3.0] * H, [2.0 ** -20] * H])
    np.testing.assert_array_equal(O.rms_norm(h, np.ones(H), 0.0, recipe), np.sign(h))
    # an all-zero row stays zero when eps > 0 (no NaN)
    assert np.array_equal(O.rms_norm(np.zeros((2, H)), np.ones(H), 1e-6, recipe), np.zeros((2, H)))
    # scale invariance: multiplying a row by a power of two changes nothing (eps = 0)
    rng = np.random.default_rng(16)
    r = rng.standard_normal((5, H)).astype(F32).astype(np.float64)
    w = 1.0 + 0.1 * rng.standard_normal(H)
    np.testing.assert_array_equal(O.rms_norm(r * 8.0, w, 0.0, recipe), O.rms_norm(r, w, 0.0, recipe))


def test_rms_norm_has_unit_rms_and_applies_the_weight_per_channel():
    rng = np.random.default_rng(17)
    H = 384
    h = rng.standard_normal((20, H)) * 3.0
    x = O.rms_norm(h, np.ones(H), 0.0, O.RECIPE_F32)
    np.testing.assert_allclose(np.sqrt((x * x).mean(axis=1)), 1.0, rtol=1e-6)
    w = 1.0 + 0.1 * rng.standard_normal(H)
    np.testing.assert_allclose(O.rms_norm(h, w, 0.0, O.RECIPE_F32), x * w[None, :], rtol=2e-7)
    # eps enters under the root: a row with mean square m gets the factor 1/sqrt(m + eps)
    xe = O.rms_norm(h, np.ones(H), 0.5, O.RECIPE_F32)
    m = (h * h).mean(axis=1)
    np.testing.assert_allclose(xe, h / np.sqrt(m + 0.5)[:, None], rtol=2e-7)


# ------------------------------------------------------------------ NVFP4
def test_encode_e2m1_grid_ties_and_saturation():
    # every code round-trips (the sign bit of zero included)
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(O.encode_e2m1(O.E2M1_TABLE[codes]), codes)
    # midpoints go to the even code; beyond 6 saturates
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.25, -5.0])
    assert O.encode_e2m1(mids).tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 7, 8, 14]
    # nearest on a fine sweep, against a brute-force search over the grid
    v = np.linspace(-7, 7, 2801)
    got = O.E2M1_TABLE[O.encode_e2m1(v)]
    grid = O.E2M1_TABLE[:8]
    for x, g in zip(v, got):
        target = min(abs(x), 6.0)
        assert abs(abs(g) - target) == np.abs(grid - target).min()      # a nearest grid value
        assert np.sign(g) in (0.0, np.sign(x))


def test_nvfp4_quantiser_scale_rule_bounds_and_fp16_exactness():
    page = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))["nvfp4"]
    assert page["group_size"] == 16 and page["scale_format"] == "FP8"
    rng = np.random.default_rng(18)
    v = (rng.standard_normal((64, 256)) * 10.0 ** rng.uniform(-3, 2, (64, 1))).astype(F32)
    v[3, 16:32] = 0.0                                   # an all-zero group: scale 1, codes 0
    v[5, :16] = 0.0; v[5, 7] = 6 * 0.5                  # amax = 6 * 2^-1: the scale is exactly 0.5
    q, sc = O.quant_nvfp4(v)
    assert q.shape == v.shape and sc.shape == (64, 256 // page["group_size"])
    s = O.decode_e4m3(sc)
    assert s[3, 1] == 1.0 and np.all(q[3, 16:32] % 8 == 0)
    assert s[5, 0] == 0.5 and O.E2M1_TABLE[q[5, 7]] == 6.0
    # the scale is the e4m3 value nearest to amax/6
    amax = np.abs(v.reshape(64, 16, 16)).max(axis=2)
    nz = amax > 0
    want = O.decode_e4m3(O.encode_e4m3((amax / F32(6)).astype(F32)))
    assert np.array_equal(s[nz], np.where(want[nz] == 0, 1.0, want[nz]))
    dq = O.dequant_nvfp4(q, sc)
    # error: at most half the e2m1 gap at the value (gaps 0.5, 1, 2), or the clip to 6*s
    x = np.abs(v.astype(np.float64)) / np.repeat(s, 16, axis=1)
    gap = np.where(x < 2, 0.5, np.where(x < 4, 1.0, 2.0))
    err = np.abs(v - dq) / np.repeat(s, 16, axis=1)
    assert np.all(err <= np.maximum(gap / 2, x - 6.0) + 1e-12)
    # every dequantised value is exact in fp16 (and bf16): the GPU multiplies them as such
    assert np.array_equal(dq.astype(np.float16).astype(np.float64), dq)
    assert np.array_equal(O.decode_bf16(O.encode_bf16(dq.astype(F32))), dq)


@pytest.mark.parametrize("recipe", [O.RECIPE_FP8_B128, O.RECIPE_MXFP4, O.RECIPE_NVFP4])
def test_quantised_recipes_quantise_the_expert_inputs(recipe):
    """The routed experts see the recipe's quantised activations: the quantiser is
    idempotent, so feeding already-quantised rows changes no expert output (with the
    same routing), while a layer that skipped the quantisation would differ."""
    cfg = {O.RECIPE_FP8_B128: C.MINI_FP8, O.RECIPE_MXFP4: C.MINI_MXFP4, O.RECIPE_NVFP4: C.MINI_NVFP4}[recipe]
    inp = G.generate(cfg)
    from tests import harness as HN
    x = HN.x_f64(inp)
    gw, b = inp.gate_w.double().numpy(), inp.bias.numpy()
    s13, s2 = HN.shared_f64(inp)
    tokens = np.arange(12)
    r1 = O.moe_forward(cfg, x, gw, b, HN.expert_raw_fn(inp), s13, s2, tokens=tokens)
    xq = O.quantize_rows(recipe, x.astype(F32))
    assert np.abs(xq - x).max() > 0                                   # the quantisation is not a no-op
    r2 = O.moe_forward(cfg, xq, gw, b, HN.expert_raw_fn(inp), s13, s2, tokens=tokens, routing=r1["routing"])
    np.testing.assert_array_equal(r1["y"], r2["y"])


# ------------------------------------------------------------------ selection key (R3)
def test_selection_key_is_the_fp32_sum_and_fp32_ties_go_to_the_lower_index():
    """The walk-through (section 3.2) adds e_score_correction_bias to each score;
    R3 takes that sum in fp32.  Two experts whose exact sums differ by 2^-30 tie in
    fp32 (half an ulp near 0.7 is 3e-8), so the lower index must win; a key kept in
    fp64 would pick the higher one."""
    s = np.array([[0.6, 0.7, 0.7, 0.1, 0.3]], dtype=F32)
    b = np.array([0.0, 0.0, 2.0 ** -30, -0.1, 0.25], dtype=F32)
    key = O.selection_key(s, b)
    for e in range(5):
        assert key[0, e] == fp32_nearest(Fraction(float(s[0, e])) + Fraction(float(b[e])))
    assert key[0, 1] == key[0, 2]
    # the same tie through the router: experts 1 and 2 have the same gate row
    cfg = rand_small_cfg(num_tokens=16, hidden=32, num_experts=8, top_k=1)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 32)).astype(F32).astype(np.float64)
    gw = (rng.standard_normal((8, 32)) * 0.01).astype(F32).astype(np.float64)
    gw[1] = gw[2] = 0.05                            # equal rows that dominate for positive x
    x = np.abs(x)
    bias = np.zeros(8, dtype=F32)
    bias[2] = F32(2.0 ** -30)
    r = O.route(cfg, x, gw, bias)
    assert np.all(r["key"][:, 1] == r["key"][:, 2])
    assert np.all(r["idx"][:, 0] == 1)


# ------------------------------------------------------------------ quantised expert path (R7, R13)
def _e4m3_value(v: float) -> float:
    """e4m3fn rounding of an fp32 value by torch's cast, saturating at 448 (R7)."""
    v = max(-448.0, min(448.0, v))
    return float(torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64))


_E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e2m1_value(v: float) -> float:
    """Nearest e2m1 grid value, ties to the even code, saturating at 6 (sign kept)."""
    a = min(abs(v), 6.0)
    best = min(range(8), key=lambda c: (abs(_E2M1_GRID[c] - a), c % 2))
    return math.copysign(_E2M1_GRID[best], v)


def _quant_row_loops(recipe: int, row32) -> list:
    """One fp32 row quantised and dequantised block by block, written from R7 / R13."""
    out = []
    if recipe == O.RECIPE_FP8_B128:
        for b0 in range(0, len(row32), 128):
            blk = [float(v) for v in row32[b0:b0 + 128]]
            amax = max(abs(v) for v in blk)
            s = float(F32(amax) / F32(448.0)) if amax > 0 else 1.0
            out += [_e4m3_value(float(F32(v) / F32(s))) * s for v in blk]
    elif recipe == O.RECIPE_MXFP4:                     # MXFP8 activations
        for b0 in range(0, len(row32), 32):
            blk = [float(v) for v in row32[b0:b0 + 32]]
            amax = max(abs(v) for v in blk)
            e = 0
            if amax > 0:
                e = -200
                while amax > 448.0 * 2.0 ** e:
                    e += 1
            e = max(-127, min(127, e))
            out += [_e4m3_value(v * 2.0 ** -e) * 2.0 ** e for v in blk]
    elif recipe == O.RECIPE_NVFP4:
        for b0 in range(0, len(row32), 16):
            blk = [float(v) for v in row32[b0:b0 + 16]]
            amax = max(abs(v) for v in blk)
            s = _e4m3_value(float(F32(amax) / F32(6.0)))
            s = s if s > 0 else 1.0
            out += [_e2m1_value(float(F32(v) / F32(s))) * s for v in blk]
    else:
        raise ValueError(recipe)
    return out


def _mlp_loops(xrow, w13, w2, quant_recipe=None):
    """SwiGLU MLP of one row with math.fsum dot products; h quantised per recipe."""
    I = w13.shape[0] // 2
    g = [math.fsum(w13[i, k] * xrow[k] for k in range(len(xrow))) for i in range(I)]
    u = [math.fsum(w13[I + i, k] * xrow[k] for k in range(len(xrow))) for i in range(I)]
    h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    if quant_recipe is not None:
        h = _quant_row_loops(quant_recipe, np.array(h).astype(F32))
    return [math.fsum(w2[o, i] * h[i] for i in range(I)) for o in range(w2.shape[0])]


@pytest.mark.parametrize("recipe", [O.RECIPE_FP8_B128, O.RECIPE_MXFP4, O.RECIPE_NVFP4])
def test_quantised_layer_matches_scalar_loops(recipe):
    """A tiny quantised layer against loops written from R7 / R13: the routed
    experts see x and h quantised per (row, 128) fp8 / (row, 32) MXFP8 / (row, 16)
    NVFP4 blocks, while the shared expert sees the unquantised x (walk-through
    section 4: shared experts stay high precision).  A wrong block size, a missed
    h quantisation or a quantised shared input all move the result by about 1e-2."""
    base = {O.RECIPE_FP8_B128: C.MINI_FP8, O.RECIPE_MXFP4: C.MINI_MXFP4, O.RECIPE_NVFP4: C.MINI_NVFP4}[recipe]
    cfg = base.replace(name="pin_" + base.name, num_tokens=3, hidden=256, intermediate=128, num_experts=4,
                       top_k=2, num_shared=1, shared_intermediate=128, n_group=1, topk_group=1)
    inp = G.generate(cfg)
    from tests import harness as HN
    x = HN.x_f64(inp)
    gw, b = inp.gate_w.double().numpy(), inp.bias.numpy()
    s13, s2 = HN.shared_f64(inp)
    raw = HN.expert_raw_fn(inp)
    got = O.moe_forward(cfg, x, gw, b, raw, s13, s2)
    idx, w = got["routing"]["idx"], got["routing"]["w"].astype(np.float64)
    for t in range(cfg.num_tokens):
        xq = _quant_row_loops(recipe, x[t].astype(F32))
        want = np.zeros(cfg.hidden)
        for j in range(cfg.top_k):
            w13, w2 = O.dequant_expert(recipe, raw(int(idx[t, j])), cfg.intermediate, cfg.hidden)
            want += w[t, j] * np.array(_mlp_loops(xq, w13, w2, quant_recipe=recipe))
        want += np.array(_mlp_loops(list(x[t]), s13[0], s2[0]))
        np.testing.assert_allclose(got["out"][t], want, rtol=1e-9, atol=1e-12)


def test_nvfp4_weight_dequantisation_against_the_source_weights():
    """NVFP4 (walk-through section 4: 4-bit weights, one FP8 scale per 16): the
    dequantised weights lie within half an e2m1 step (times the group scale) of the
    fp32 source values, except where the group's largest value saturates at 6 x
    scale; each scale is the e4m3 value nearest to amax / 6."""
    g = torch.Generator().manual_seed(3)
    w = torch.randn(64, 256, generator=g) * 0.02
    w[5, 16:32] = 0.0
    q, sc = G.encode_nvfp4(w)
    d = O.dequant_expert(C.RECIPE_NVFP4, {"w13": q.numpy(), "w13_scale": sc.numpy(),
                                         "w2": q.numpy(), "w2_scale": sc.numpy()}, 32, 256)[0]
    ref = w.double().numpy()
    s = np.array([[_e4m3_value(float(F32(a) / F32(6.0))) or 1.0 for a in row]
                  for row in np.abs(ref).reshape(64, 16, 16).max(axis=2)])
    np.testing.assert_array_equal(O.decode_e4m3(sc.numpy()), s)
    sfull = np.repeat(s, 16, axis=1)
    a = np.abs(ref) / sfull
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = 0.5 * step * sfull + np.maximum(0.0, np.abs(ref) - 6.0 * sfull)
    assert np.all(np.abs(d - ref) <= bound + 1e-30)
    assert np.all(d[5, 16:32] == 0.0)


def test_residual_form_matches_scalar_loops():
    """Decoder-layer residual form (walk-through section 3.5): out = h + MoE(x) with
    x = RMSNorm(h) per row, (h * r) * weight, r = 1 / sqrt(mean(h^2) + eps), rounded
    to fp32 and then to bf16 (R12).  The norm is written here with math.fsum and
    torch's bf16 cast; the MoE part is the oracle's own (pinned above)."""
    cfg = C.MINI_GROUPED_BF16.replace(name="pin_resid", num_tokens=5)
    inp = G.generate(cfg)
    from tests import harness as HN
    h = HN.x_f64(inp)
    nw = (1.0 + 0.1 * np.random.default_rng(4).standard_normal(cfg.hidden)).astype(F32)
    eps = 1e-6
    x = np.empty_like(h)
    for t in range(cfg.num_tokens):
        r = 1.0 / math.sqrt(math.fsum(v * v for v in h[t]) / cfg.hidden + eps)
        y32 = torch.tensor([(v * r) * float(wv) for v, wv in zip(h[t], nw)], dtype=torch.float64).to(torch.float32)
        x[t] = y32.to(torch.bfloat16).to(torch.float64).numpy()
    gw, b = inp.gate_w.double().numpy(), inp.bias.numpy()
    s13, s2 = HN.shared_f64(inp)
    got = O.moe_forward_residual(cfg, h, nw, eps, gw, b, HN.expert_raw_fn(inp), s13, s2)
    np.testing.assert_array_equal(got["x"], x)
    plain = O.moe_forward(cfg, x, gw, b, HN.expert_raw_fn(inp), s13, s2)
    np.testing.assert_array_equal(got["out"], h + plain["out"])
    # token subset: rows line up with their residual rows
    sub = O.moe_forward_residual(cfg, h, nw, eps, gw, b, HN.expert_raw_fn(inp), s13, s2, tokens=np.array([4, 1]))
    np.testing.assert_allclose(sub["out"], got["out"][[4, 1]], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ FP4 -> FP8 conversion (R14)
def _mx_block(rng, rows=128, cols=256, spread=3):
    """Random MXFP4 weights whose per-32 exponents (E8M0 bytes) span `spread` + 1 values."""
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    e8 = (120 + rng.integers(0, spread + 1, (rows, cols // 32))).astype(np.uint8)
    return packed, e8


def test_mxfp4_to_fp8_is_lossless_within_an_exponent_spread_of_8():
    """V4-Pro overview, convert.py: the FP4 -> FP8 conversion is lossless.  With the
    groups of every 128 x 128 block within 8 binades, each converted value times its
    block scale equals the MXFP4 value exactly (MX dequantisation, pinned above)."""
    rng = np.random.default_rng(11)
    packed, e8 = _mx_block(rng, 256, 384, spread=8)
    codes, scales, bad = O.convert_mxfp4_to_fp8(packed, e8)
    assert bad == 0
    want = O.dequant_expert(C.RECIPE_MXFP4, {"w13": packed, "w13_scale": e8, "w2": packed, "w2_scale": e8}, 128, 384)[0]
    got = O.decode_e4m3(codes) * np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)
    np.testing.assert_array_equal(got, want)
    # the fp8 recipe's own dequantisation reads the converted weights as the same values
    fp8 = O.dequant_expert(C.RECIPE_FP8_B128, {"w13": codes, "w13_scale": scales, "w2": codes, "w2_scale": scales},
                           128, 384)[0]
    np.testing.assert_array_equal(fp8, want)


def test_mxfp4_to_fp8_rounds_and_counts_blocks_beyond_the_spread():
    """A block whose groups span more than 8 binades cannot keep its smallest values:
    they round to the nearest e4m3 value (ties to even, checked against an exact
    brute-force search with fractions) and the block is counted."""
    rng = np.random.default_rng(12)
    packed, e8 = _mx_block(rng, 128, 256, spread=2)
    e8[5, 1] = 110                                   # 10 and more binades below the block maximum
    e8[9, 6] = 100
    codes, scales, bad = O.convert_mxfp4_to_fp8(packed, e8)
    assert bad >= 1
    pos = [Fraction(float(v)) for v in O.E4M3_TABLE[:0x7F]]
    v = O.decode_e2m1_packed(packed)
    for r, g in ((5, 1), (9, 6)):
        E = int(e8[(r // 128) * 128:(r // 128 + 1) * 128, (g // 4) * 4:(g // 4 + 1) * 4].max())
        for c in range(32 * g, 32 * g + 32):
            x = Fraction(float(v[r, c])) * Fraction(2) ** (int(e8[r, g]) - E)
            ranked = sorted(range(len(pos)), key=lambda i: (abs(pos[i] - abs(x)), i % 2))
            want = float(pos[ranked[0]]) * (-1.0 if math.copysign(1.0, float(v[r, c])) < 0 else 1.0)
            assert O.decode_e4m3(codes[r:r + 1, c:c + 1])[0, 0] == want
