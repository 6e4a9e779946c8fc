"""CPU oracle for the DeepSeek-V3-style MoE layer forward.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the GPU library: every decoder,
encoder, score function, selection rule, permutation and product below is
written here, in numpy float64 (float32 where a step is defined in fp32), with
numpy's matmul and stable argsort as the only library primitives.

What it computes follows the Kimi-K2-Thinking-NVFP4 walk-through of the
DeepSeek-V3 architecture (pwwt.cn/news/5781524), section 3 "MoE routing":
  3.1 scoring   - the gate matrix [E, H] times the hidden state in FP32, then an
                  independent sigmoid per expert;
  3.2 selection - noaux_tc: add e_score_correction_bias to every score; per
                  group, sum the two best scores; keep topk_group groups; take
                  the top-k experts among the kept candidates;
  3.3 weights   - the k selected scores normalised to sum 1
                  (norm_topk_prob), times routed_scaling_factor;
  3.4 moe_infer - count tokens per expert, argsort tokens by expert id into
                  contiguous blocks, run each expert's gate/up/down + SiLU MLP
                  on its block, put rows back in the original order, multiply
                  by the top-k weights and sum; add the shared expert, which
                  sees every token.
The DeepSeek-V4-Pro overview (lzwjava.github.io, "architecture" and
"model.py") adds the sqrtsoftplus score and route_scale; its "kernel.py"
entry gives fp8 activation blocks of 128 and FP4 blocks of 32 with
power-of-two scales; the 2.8T articles (ruibaoantu.com, "quantisation") give
MXFP4 weights with MXFP8 activations.

Readings taken where the pages are silent or garbled (each is listed with its
reason in the design notes):
  R1 logits: the FP32 logit is the fp32 rounding (nearest-even) of the
     dot product evaluated in fp64 with exact products.
  R2 scores: s = fp32(f(fp32 logit)) with f evaluated in fp64;
     sqrtsoftplus(z) = sqrt(log(1 + e^z)).
  R3 selection key: key = fp32(s + bias); total order key descending, then
     expert index ascending; NaN ranks below every number.
  R4 groups: n_group contiguous groups; group score = fp32 sum of the group's
     two largest keys (biased); keep the topk_group best groups (ties: lower
     group index); experts of dropped groups are excluded from the top-k.
  R5 weights use the unbiased scores s of the selected experts; fp64
     normalisation, result rounded to fp32; no epsilon.
  R6 the argsort is stable: rows of one expert appear in increasing flat
     pair index f = t*k + j.
  R7 activation quantisation (fp8/MX recipes) applies to the rows fed to the
     routed experts (x and the SwiGLU output h, both as fp32 values):
       fp8 per (row, 128 channels): s = fp32(amax/448), q = e4m3(fp32(v/s));
       MXFP8 per (row, 32 channels): e = least integer with amax <= 448*2^e,
       q = e4m3(v * 2^-e); an all-zero block takes scale 1 (e = 0).
     e4m3 encoding rounds to nearest, ties to even code, saturating at 448,
     and keeps the input's sign bit (a negative value that rounds to zero
     gives the code 0x80).
     The shared experts and the gate see the unquantised x.
  R8 FFN in fp64 on the dequantised weights; no bias; shared experts are
     summed; the output excludes the residual (the residual form below adds it).
  R11 swiglu_limit (V4-Pro overview, FFN entry, named only): when > 0, every
     SwiGLU computes SiLU(min(g, L)) * clamp(u, -L, L).
  R12 residual form (walk-through 3.5 decoder layer; V4-Pro overview: RMSNorm
     kept in fp32): x = post_attention_layernorm(h) with each row
     (h * r) * weight, r = 1/sqrt(mean(h^2) + eps), evaluated in fp64, rounded to
     fp32 and then to the activation format; out = h + MoE(x).
  R13 NVFP4 (walk-through section 4: 4-bit floats for routed-expert weights and
     their input activations, one FP8 scale per 16 values; shared experts stay
     high precision): per (row, 16 consecutive input channels)
       s = e4m3(fp32(amax / 6)), taken as 1 when that rounds to 0,
       q = e2m1(fp32(v / s)) rounding to nearest, ties to even code,
           saturating at 6 and keeping the sign bit;
     the value is q * s.  No per-tensor scale (the page names none).  The
     activations are the rows fed to the routed experts (x and h), as in R7.
  R14 FP4 -> FP8 conversion (V4-Pro overview, convert.py: lossless e2m1fn to
     e4m3fn with care for the scales): MXFP4 weights become e4m3fn codes with one
     fp32 scale per 128 x 128 block, 2^(largest E8M0 exponent of the block's
     groups); see convert_mxfp4_to_fp8.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
F64 = np.float64

SCORE_SIGMOID = 0
SCORE_SQRTSOFTPLUS = 1

RECIPE_F32, RECIPE_BF16, RECIPE_FP8_B128, RECIPE_MXFP4, RECIPE_NVFP4 = 0, 1, 2, 3, 4


# =============================================================== number formats
def decode_bf16(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the upper half of an fp32."""
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(F64)


def encode_bf16(v32: np.ndarray) -> np.ndarray:
    """Finite fp32 values -> bfloat16 bit patterns, rounding to nearest, ties to even."""
    u = np.ascontiguousarray(v32, dtype=F32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def _e4m3fn_table() -> np.ndarray:
    """OCP FP8 E4M3 ('fn': no infinities, S.1111.111 is NaN): bias 7, 3 mantissa bits."""
    t = np.empty(256, dtype=F64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = math.nan
        elif e == 0:
            t[c] = s * m * 2.0 ** (-9)          # subnormal: m/8 * 2^-6
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _e4m3fn_table()
E4M3_MAX = 448.0

# E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                       -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=F64)


def decode_e4m3(u8: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[u8.astype(np.int64)]


def decode_e2m1_packed(u8: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes, low nibble = even k -> float64 [..., K]."""
    lo = E2M1_TABLE[(u8 & 0xF).astype(np.int64)]
    hi = E2M1_TABLE[(u8 >> 4).astype(np.int64)]
    out = np.empty(u8.shape[:-1] + (u8.shape[-1] * 2,), dtype=F64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# positive e2m1 values in code order 0..7 and the midpoints between neighbours
_E2M1_POS = E2M1_TABLE[:8]
_E2M1_MID = (_E2M1_POS[:-1] + _E2M1_POS[1:]) / 2.0


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Round values to e2m1 codes (0..15): nearest, ties to the even code, saturate at 6;
    the sign bit is kept (a negative value that rounds to zero gives code 8)."""
    a = np.abs(np.asarray(v, dtype=F64))
    below = (a[..., None] > _E2M1_MID).sum(axis=-1)            # midpoints strictly below
    tie = (a[..., None] == _E2M1_MID)
    # on a tie between codes i and i+1 (midpoint i), take the even one
    tie_idx = np.where(tie.any(axis=-1), tie.argmax(axis=-1), -1)
    code = np.where(tie_idx >= 0, np.where(tie_idx % 2 == 0, tie_idx, tie_idx + 1), below)
    sign = (np.signbit(np.asarray(v, dtype=F64))).astype(np.int64) << 3
    return (code + sign).astype(np.uint8)


def decode_e8m0(u8: np.ndarray) -> np.ndarray:
    """E8M0 scale byte: 2^(b - 127); 0xFF is NaN."""
    b = u8.astype(np.int64)
    v = np.ldexp(1.0, b - 127).astype(F64)
    return np.where(b == 255, math.nan, v)


# positive finite e4m3 values in code order 0x00..0x7E (increasing)
_E4M3_POS = E4M3_TABLE[:0x7F]
_E4M3_MID = (_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2.0      # exact in fp64


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Round values (fp32 or fp64) to e4m3fn codes: nearest, ties to even code, saturate at 448."""
    a = np.abs(v.astype(F64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # i = number of midpoints strictly below a -> candidate code; fix ties to even
    i = np.searchsorted(_E4M3_MID, a, side="left")
    tie = (i < len(_E4M3_MID)) & (a == _E4M3_MID[np.minimum(i, len(_E4M3_MID) - 1)])
    i = np.where(tie & (i % 2 == 1), i + 1, i)   # at a tie a is at mid[i]: codes i and i+1; pick even
    code = i.astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7      # the sign is kept, also when the result is zero
    return np.where(nan, np.uint8(0x7F), code | sign).astype(np.uint8)


# =============================================================== routing (MoEGate)
def gate_logits(x64: np.ndarray, gate_w64: np.ndarray) -> np.ndarray:
    """R1: fp32 rounding of the fp64 dot products (products of fp32/bf16 values are exact in fp64)."""
    return (x64 @ gate_w64.T).astype(F32)


def score(logits32: np.ndarray, func: int) -> np.ndarray:
    """R2: per-expert score, evaluated in fp64 from the fp32 logit, rounded to fp32."""
    z = logits32.astype(F64)
    if func == SCORE_SIGMOID:
        ez = np.exp(-np.abs(z))
        s = np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))
    elif func == SCORE_SQRTSOFTPLUS:
        sp = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
        s = np.sqrt(sp)
    else:
        raise ValueError(func)
    return s.astype(F32)


def selection_key(s32: np.ndarray, bias32: np.ndarray) -> np.ndarray:
    """R3: key = fp32(s + bias); -0 becomes +0 (adding +0.0); NaN ranks lowest."""
    key = (s32.astype(F32) + bias32.astype(F32)[None, :]) + F32(0.0)
    return np.where(np.isnan(key), F32(-np.inf), key).astype(F32)


def _order_desc(values: np.ndarray) -> np.ndarray:
    """Per row: indices sorted by value descending, ties by index ascending (stable sort of -v)."""
    return np.argsort(-values.astype(F64), axis=-1, kind="stable")


def group_mask(key32: np.ndarray, n_group: int, topk_group: int):
    """R4: returns (kept [T, E] bool, group scores [T, n_group] fp32)."""
    T, E = key32.shape
    if n_group == 1:
        return np.ones((T, E), dtype=bool), key32.max(axis=1, keepdims=True)
    gsz = E // n_group
    g = key32.reshape(T, n_group, gsz)
    top2 = np.sort(g.astype(F64), axis=-1)[..., -2:]               # two largest keys per group
    gscore = (top2[..., 1].astype(F32) + top2[..., 0].astype(F32)).astype(F32)
    gorder = _order_desc(gscore)[:, :topk_group]
    keep_g = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(keep_g, gorder, True, axis=1)
    return np.repeat(keep_g, gsz, axis=1), gscore


def route(cfg, x64: np.ndarray, gate_w64: np.ndarray, bias32: np.ndarray):
    """MoEGate.forward: returns dict(idx [T,k] int32, w [T,k] fp32, logits, s, key, kept)."""
    logits = gate_logits(x64, gate_w64)
    s = score(logits, cfg.score_func)
    key = selection_key(s, bias32)
    kept, gscore = group_mask(key, cfg.n_group, cfg.topk_group)
    T, E = key.shape
    # total order: kept first, then key descending, then index ascending
    o1 = _order_desc(np.where(kept, key, F32(-np.inf)))
    excl = ~np.take_along_axis(kept, o1, axis=1)
    o2 = np.argsort(excl, axis=1, kind="stable")
    order = np.take_along_axis(o1, o2, axis=1)
    idx = order[:, :cfg.top_k].astype(np.int32)
    sel = np.take_along_axis(s, idx, axis=1).astype(F64)
    if cfg.norm_topk_prob:
        w = sel / sel.sum(axis=1, keepdims=True) * float(cfg.routed_scaling_factor)
    else:
        w = sel * float(cfg.routed_scaling_factor)
    return dict(idx=idx, w=w.astype(F32), logits=logits, s=s, key=key, kept=kept,
                gscore=gscore, order=order)


def boundary_gap(key32: np.ndarray, order: np.ndarray, k: int) -> np.ndarray:
    """Per token: key of the k-th pick minus the (k+1)-th candidate, in fp64 (diagnostic)."""
    kk = np.take_along_axis(key32, order, axis=1).astype(F64)
    if kk.shape[1] <= k:
        return np.full(kk.shape[0], np.inf)
    return kk[:, k - 1] - kk[:, k]


# =============================================================== permutation (moe_infer)
def permute(idx: np.ndarray, num_experts: int):
    """R6: counts, offsets [E+1], sorted_pair [T*k] (row -> flat pair f), pair_pos [T*k] (f -> row)."""
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int32)
    pair_pos = np.empty_like(sorted_pair)
    pair_pos[sorted_pair] = np.arange(flat.size, dtype=np.int32)
    return dict(counts=counts, offsets=offsets, sorted_pair=sorted_pair, pair_pos=pair_pos)


# =============================================================== activation quantisation
def quant_fp8_b128(v32: np.ndarray):
    """R7 fp8: per (row, 128 channels). Returns (codes uint8 [R, C], scales fp32 [R, C/128])."""
    R, Cn = v32.shape
    b = v32.astype(F32).reshape(R, Cn // 128, 128)
    amax = np.abs(b).max(axis=2)
    s = np.where(amax > 0, (amax / F32(E4M3_MAX)).astype(F32), F32(1.0)).astype(F32)
    q = encode_e4m3((b / s[:, :, None]).astype(F32))
    return q.reshape(R, Cn), s


def dequant_fp8_b128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    R, Cn = codes.shape
    return (decode_e4m3(codes).reshape(R, Cn // 128, 128) * scales.astype(F64)[:, :, None]).reshape(R, Cn)


def mx_exponent(amax: np.ndarray, elem_max: float) -> np.ndarray:
    """Least integer e with amax <= elem_max * 2^e (0 for amax == 0), clamped to [-127, 127]."""
    a = amax.astype(F64)
    e = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    # start from floor(log2(a / elem_max)) and step up until the bound holds (exact comparisons)
    _, ex = np.frexp(np.where(nz, a, 1.0) / elem_max)
    e = np.where(nz, ex - 2, 0)
    for _ in range(4):
        need_up = nz & (a > elem_max * np.ldexp(1.0, e))
        e = np.where(need_up, e + 1, e)
    return np.clip(e, -127, 127)


def quant_mxfp8(v32: np.ndarray):
    """R7 MXFP8: per (row, 32 channels). Returns (codes uint8 [R, C], E8M0 uint8 [R, C/32])."""
    R, Cn = v32.shape
    b = v32.astype(F32).reshape(R, Cn // 32, 32).astype(F64)
    amax = np.abs(b).max(axis=2)
    e = mx_exponent(amax, E4M3_MAX)
    q = encode_e4m3(b * np.ldexp(1.0, -e)[:, :, None])
    return q.reshape(R, Cn), (e + 127).astype(np.uint8)


def dequant_mxfp8(codes: np.ndarray, e8: np.ndarray) -> np.ndarray:
    R, Cn = codes.shape
    return (decode_e4m3(codes).reshape(R, Cn // 32, 32) * decode_e8m0(e8)[:, :, None]).reshape(R, Cn)


def quant_nvfp4(v32: np.ndarray):
    """R13: per (row, 16 channels). Returns (e2m1 codes uint8 [R, C], e4m3 scale codes uint8 [R, C/16])."""
    R, Cn = v32.shape
    b = v32.astype(F32).reshape(R, Cn // 16, 16)
    amax = np.abs(b).max(axis=2)
    sc = encode_e4m3((amax / F32(6.0)).astype(F32))
    sc = np.where(decode_e4m3(sc) == 0, encode_e4m3(np.array(1.0)), sc).astype(np.uint8)
    s = decode_e4m3(sc).astype(F32)
    q = encode_e2m1((b / s[:, :, None]).astype(F32))
    return q.reshape(R, Cn), sc


def dequant_nvfp4(codes: np.ndarray, scale_codes: np.ndarray) -> np.ndarray:
    R, Cn = codes.shape
    return (E2M1_TABLE[codes.astype(np.int64)].reshape(R, Cn // 16, 16)
            * decode_e4m3(scale_codes)[:, :, None]).reshape(R, Cn)


def quantize_rows(recipe: int, v: np.ndarray):
    """Quantise-dequantise rows per the recipe's activation format (identity for f32/bf16)."""
    if recipe == RECIPE_FP8_B128:
        q, s = quant_fp8_b128(v.astype(F32))
        return dequant_fp8_b128(q, s)
    if recipe == RECIPE_MXFP4:
        q, e = quant_mxfp8(v.astype(F32))
        return dequant_mxfp8(q, e)
    if recipe == RECIPE_NVFP4:
        q, s = quant_nvfp4(v.astype(F32))
        return dequant_nvfp4(q, s)
    return v.astype(F64)


# =============================================================== weights
def dequant_expert(recipe: int, raw: dict, I: int, H: int):
    """raw: numpy views of one expert's stored weights -> (w13 [2I, H], w2 [H, I]) fp64.

    raw keys: w13, w2 (float32 / uint16 bf16 bits / uint8 e4m3 / uint8 packed e2m1),
              w13_scale, w2_scale (fp32 128x128 block scales, uint8 E8M0 per 32, or
              uint8 e4m3 per 16 for NVFP4)."""
    if recipe == RECIPE_F32:
        return raw["w13"].astype(F64), raw["w2"].astype(F64)
    if recipe == RECIPE_BF16:
        return decode_bf16(raw["w13"]), decode_bf16(raw["w2"])
    if recipe == RECIPE_FP8_B128:
        def blk(q, s):
            R, K = q.shape
            return (decode_e4m3(q).reshape(R // 128, 128, K // 128, 128)
                    * s.astype(F64)[:, None, :, None]).reshape(R, K)
        return blk(raw["w13"], raw["w13_scale"]), blk(raw["w2"], raw["w2_scale"])
    if recipe == RECIPE_MXFP4:
        def mx(q, e8):
            v = decode_e2m1_packed(q)
            R, K = v.shape
            return (v.reshape(R, K // 32, 32) * decode_e8m0(e8)[:, :, None]).reshape(R, K)
        return mx(raw["w13"], raw["w13_scale"]), mx(raw["w2"], raw["w2_scale"])
    if recipe == RECIPE_NVFP4:
        def nv(q, sc):
            v = decode_e2m1_packed(q)
            R, K = v.shape
            return (v.reshape(R, K // 16, 16) * decode_e4m3(sc)[:, :, None]).reshape(R, K)
        return nv(raw["w13"], raw["w13_scale"]), nv(raw["w2"], raw["w2_scale"])
    raise ValueError(recipe)


def silu(z: np.ndarray) -> np.ndarray:
    ez = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))
    return z * sig


def swiglu(g: np.ndarray, u: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """SiLU(g) * u.  With swiglu_limit > 0 (V4-Pro overview, FFN entry: an optional
    truncation of the SwiGLU), the gate is first clamped to at most the limit and the
    up projection to [-limit, limit] (reading: the pages give only the name)."""
    if limit > 0:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    return silu(g) * u


def expert_mlp(x64: np.ndarray, w13: np.ndarray, w2: np.ndarray, recipe: int = RECIPE_F32,
               quantize_h: bool = False, limit: float = 0.0) -> np.ndarray:
    """DeepseekV3MLP on a block of rows: down(SiLU(gate(x)) * up(x)); fp64."""
    I = w13.shape[0] // 2
    g = x64 @ w13[:I].T
    u = x64 @ w13[I:].T
    h = swiglu(g, u, limit)
    if quantize_h:
        h = quantize_rows(recipe, h.astype(F32))
    return h @ w2.T


# =============================================================== the layer
def moe_forward(cfg, x64: np.ndarray, gate_w64: np.ndarray, bias32: np.ndarray,
                expert_raw, shared_w13: np.ndarray, shared_w2: np.ndarray,
                tokens: np.ndarray | None = None, routing=None, perm=None):
    """DeepseekV3MoE.forward over all tokens, or over the subset `tokens` (routing and
    the permutation are always computed for every token).

    expert_raw(e) -> raw dict for dequant_expert.  shared_w13 [S, 2Is, H] and
    shared_w2 [S, H, Is] are fp64.  Returns dict with out [len(tokens), H] fp64,
    y rows per (token, slot), routing and permutation."""
    T, H, k, E = cfg.num_tokens, cfg.hidden, cfg.top_k, cfg.num_experts
    I = cfg.intermediate
    recipe = cfg.recipe
    quant = recipe in (RECIPE_FP8_B128, RECIPE_MXFP4, RECIPE_NVFP4)
    limit = float(getattr(cfg, "swiglu_limit", 0.0))
    if routing is None:
        routing = route(cfg, x64, gate_w64, bias32)
    if perm is None:
        perm = permute(routing["idx"], E)
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    idx = routing["idx"][tokens]                                   # [n, k]
    w = routing["w"][tokens].astype(F64)
    xa = x64[tokens]
    xq = quantize_rows(recipe, xa.astype(F32)) if quant else xa   # routed experts' input rows
    y = np.zeros((len(tokens), k, H), dtype=F64)
    # moe_infer order: expert by expert over its block of (token, slot) pairs
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        w13, w2 = dequant_expert(recipe, expert_raw(int(e)), I, H)
        y[rows, slots] = expert_mlp(xq[rows], w13, w2, recipe, quantize_h=quant, limit=limit)
    routed = np.einsum("nk,nkh->nh", w, y)
    shared = np.zeros_like(routed)
    for s in range(shared_w13.shape[0]):
        shared += expert_mlp(xa, shared_w13[s], shared_w2[s], limit=limit)
    return dict(out=routed + shared, y=y, routed=routed, shared=shared, routing=routing,
                perm=perm, tokens=tokens)


def rms_norm(h: np.ndarray, weight: np.ndarray, eps: float, recipe: int) -> np.ndarray:
    """post_attention_layernorm over the rows of the residual stream h (R12).
    Returns the stored rows' values as float64 (fp32 values, or bf16 values for the
    other recipes)."""
    h64 = np.asarray(h, dtype=F64)
    r = 1.0 / np.sqrt((h64 * h64).sum(axis=1) / h64.shape[1] + float(eps))
    y32 = ((h64 * r[:, None]) * np.asarray(weight, dtype=F64)[None, :]).astype(F32)
    if recipe == RECIPE_F32:
        return y32.astype(F64)
    return decode_bf16(encode_bf16(y32))


def moe_forward_residual(cfg, h64: np.ndarray, norm_w: np.ndarray, eps: float, gate_w64: np.ndarray,
                         bias32: np.ndarray, expert_raw, shared_w13: np.ndarray, shared_w2: np.ndarray,
                         tokens: np.ndarray | None = None):
    """The decoder layer's MoE half (walk-through 3.5): out = h + MoE(RMSNorm(h))."""
    x = rms_norm(h64, norm_w, eps, cfg.recipe)
    r = moe_forward(cfg, x, gate_w64, bias32, expert_raw, shared_w13, shared_w2, tokens=tokens)
    r["x"] = x
    r["moe_out"] = r["out"]
    r["out"] = np.asarray(h64, dtype=F64)[r["tokens"]] + r["out"]
    return r


def gather_rows(recipe: int, x32: np.ndarray, sorted_pair: np.ndarray, k: int):
    """x_perm as the permute step stores it: rows x[sorted_pair[p] // k], quantised per recipe.
    Returns (rows, scales) with rows in storage form (fp32 / codes) and scales or None."""
    rows = x32[sorted_pair // k]
    if recipe == RECIPE_FP8_B128:
        return quant_fp8_b128(rows)
    if recipe == RECIPE_MXFP4:
        return quant_mxfp8(rows)
    if recipe == RECIPE_NVFP4:                 # stored as the (fp16-exact) values
        return quantize_rows(RECIPE_NVFP4, rows), None
    return rows, None


def mxfp4_bytes_per_param() -> float:
    """Storage of one MXFP4 parameter: a 4-bit element plus one 8-bit scale per 32."""
    return 0.5 + 1.0 / 32.0


# =============================================================== FP4 -> FP8 weight conversion
def convert_mxfp4_to_fp8(q_packed: np.ndarray, e8m0: np.ndarray):
    """MXFP4 weights -> the fp8 recipe's format (e4m3fn codes, one fp32 scale per
    128 x 128 block): the DeepSeek-V4-Pro overview's convert.py entry converts FP4
    (e2m1fn) to FP8 (e4m3fn) losslessly, with care for the scales.

    Reading (R14): the scale of block B is 2^(E_B - 127) with E_B the largest E8M0
    byte of the per-32 groups in B; an element of a group with byte b and e2m1 value q
    becomes e4m3(q * 2^(b - E_B)), rounding to nearest, ties to the even code.  Every
    e2m1 value is an e4m3 value, so the block is reproduced exactly whenever its
    groups' exponents differ by at most 8 (0.5 * 2^-8 is e4m3's smallest subnormal).
    q_packed [R, K/2] (low nibble = even k), e8m0 [R, K/32]; R, K multiples of 128.
    Returns (codes uint8 [R, K], scales fp32 [R/128, K/128], blocks not reproduced)."""
    v = decode_e2m1_packed(q_packed)
    R, K = v.shape
    b = e8m0.astype(np.int64)
    E = b.reshape(R // 128, 128, K // 128, 4).max(axis=(1, 3))
    d = np.repeat(np.repeat(E, 128, axis=0), 128, axis=1) - np.repeat(b, 32, axis=1)
    x = v * np.ldexp(1.0, -d)                           # exact in fp64
    codes = encode_e4m3(x)
    scales = np.ldexp(1.0, E - 127).astype(F32)
    exact = (decode_e4m3(codes) == x).reshape(R // 128, 128, K // 128, 128).all(axis=(1, 3))
    return codes, scales, int((~exact).sum())
