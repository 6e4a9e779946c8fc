// MoEGate.forward on gfx950: gate logits, scores, noaux_tc grouped top-k, weights.
//
// Walk-through of the DeepSeek-V3 architecture (pwwt.cn/news/5781524), section 3:
// 3.1 the gate matrix [E, H] times the hidden state in FP32, sigmoid per expert;
// 3.2 + e_score_correction_bias, group top-2 sums, keep topk_group groups, top-k;
// 3.3 normalise the k picked scores to sum 1, times routed_scaling_factor.
// sqrtsoftplus is the DeepSeek-V4-Pro score (lzwjava.github.io, architecture).
//
// Two gate paths with the same selection, that of the exact logits (the fp32
// rounding of fp64-accumulated dot products): the fp64-MFMA gate and its router
// (fp32 activations, and bf16 below 512 tokens), and the bf16-MFMA screen with an
// exact recompute of the experts its error bound leaves open (bf16, 512 tokens or
// more).
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Gate logits: logits[t][e] = fp32( sum_h x[t][h] * Wg[e][h] ), accumulated in fp64.
// Products of bf16/fp32 by fp32 values are exact in fp64, so the only rounding
// that matters is the final one to fp32: the kernel reproduces the correctly
// rounded FP32 linear layer except when the fp64 sum lands within ~1e-16
// (relative) of an fp32 rounding boundary.
//
// fp64 MFMA 16x16x4: a 128 x 64 (token x expert) tile per 256-thread block; wave w
// owns tokens 32w .. 32w+31 against all 64 experts (2 x 4 MFMA tiles).  K runs in
// chunks of 32, staged through LDS as fp32 (bf16 widens exactly) in a two-slot
// ring; the global loads (16 bytes per lane) of the next two chunks are in flight
// in two register sets while the current chunk is multiplied.  Within a chunk, lane group g = lane / 16 takes
// k = 8g .. 8g+7 over the chunk's 8 MFMA steps (the same K order for both
// operands), so that each lane reads its 8 k of a row with two 16-byte LDS reads.
// ---------------------------------------------------------------------------
constexpr int GT = 128, GE = 64, GK = 32, GPAD = GK + 4;   // 144-byte LDS rows: conflict-free 16-lane reads

template <typename XT>
struct GateLoad;
template <>
struct GateLoad<uint16_t> {                        // bf16 x: 8 values (16 bytes) per load, 2 loads per thread
  static constexpr int PER_ROW = GK / 8, N = GT * PER_ROW / 256;
  uint4 v[N];
};
template <>
struct GateLoad<float> {                           // fp32 x: 4 values per load, 4 loads per thread
  static constexpr int PER_ROW = GK / 4, N = GT * PER_ROW / 256;
  float4 v[N];
};

// Split over K (blockIdx.z) when there are too few (token, expert) tiles to fill
// the chip: each split writes fp64 partial sums, which the router adds in a fixed
// order before the single rounding to fp32.
template <typename XT>
__global__ __launch_bounds__(256) void gate_logits_f64(const XT* __restrict__ x, const float* __restrict__ wg,
                                                       float* __restrict__ logits, double* __restrict__ partial,
                                                       int T, int E, int H, int kchunk) {
  __shared__ __attribute__((aligned(16))) float As[2][GT][GPAD];
  __shared__ __attribute__((aligned(16))) float Bs[2][GE][GPAD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.y * GT, e0 = blockIdx.x * GE;
  const int kbeg = blockIdx.z * kchunk, nch = kchunk / GK;

  // global -> register loads of one chunk (rows past T / E read row 0 and store 0)
  using LA = GateLoad<XT>;
  LA las[2];                                        // two register sets: chunks c and c+1 in flight
  float4 lbs[2][2];                                 // Wg: 64 rows x 8 segments of 4 floats
  auto load = [&](int k0, auto setc) {
    LA& la = las[decltype(setc)::value];
    float4 (&lb)[2] = lbs[decltype(setc)::value];
#pragma unroll
    for (int i = 0; i < LA::N; ++i) {
      const int idx = tid + 256 * i, row = idx / LA::PER_ROW, seg = idx % LA::PER_ROW;
      const int t = min(t0 + row, T - 1);
      if constexpr (sizeof(XT) == 2) la.v[i] = *reinterpret_cast<const uint4*>(x + size_t(t) * H + k0 + seg * 8);
      else la.v[i] = *reinterpret_cast<const float4*>(x + size_t(t) * H + k0 + seg * 4);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i, row = idx / 8, seg = idx % 8;
      const int e = min(e0 + row, E - 1);
      lb[i] = *reinterpret_cast<const float4*>(wg + size_t(e) * H + k0 + seg * 4);
    }
  };
  auto store = [&](auto setc, int buf) {
    const LA& la = las[decltype(setc)::value];
    const float4 (&lb)[2] = lbs[decltype(setc)::value];
#pragma unroll
    for (int i = 0; i < LA::N; ++i) {
      const int idx = tid + 256 * i, row = idx / LA::PER_ROW, seg = idx % LA::PER_ROW;
      const bool ok = t0 + row < T;
      if constexpr (sizeof(XT) == 2) {
        const uint32_t w[4] = {la.v[i].x, la.v[i].y, la.v[i].z, la.v[i].w};
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[2 * q] = ok ? __uint_as_float(w[q] << 16) : 0.0f;
          f[2 * q + 1] = ok ? __uint_as_float(w[q] & 0xffff0000u) : 0.0f;
        }
        *reinterpret_cast<float4*>(&As[buf][row][seg * 8]) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(&As[buf][row][seg * 8 + 4]) = make_float4(f[4], f[5], f[6], f[7]);
      } else {
        *reinterpret_cast<float4*>(&As[buf][row][seg * 4]) = ok ? la.v[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i, row = idx / 8, seg = idx % 8;
      const bool ok = e0 + row < E;
      *reinterpret_cast<float4*>(&Bs[buf][row][seg * 4]) = ok ? lb[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  f64x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

  // Chunk c is multiplied from LDS slot c & 1 while chunks c+1 and c+2 are in
  // flight into register set (c+1) & 1 and c & 1; chunk c+1 goes to the other LDS
  // slot after the MFMAs.  The barrier leaves the register loads in flight (a
  // fenced __syncthreads would wait for them).
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto chunk = [&](int c, auto setc) {
    constexpr int st = decltype(setc)::value;
    // set st held chunk c, already in LDS.  Unconditional (the last chunks reload
    // chunk nch-1, unused): a conditional load makes the compiler wait for it at once.
    load(kbeg + min(c + 2, nch - 1) * GK, setc);
    float a[2][8], b[4][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* p = &As[st][wave * 32 + 16 * i + r16][8 * g];
      const float4 lo = *reinterpret_cast<const float4*>(p), hi = *reinterpret_cast<const float4*>(p + 4);
      a[i][0] = lo.x; a[i][1] = lo.y; a[i][2] = lo.z; a[i][3] = lo.w;
      a[i][4] = hi.x; a[i][5] = hi.y; a[i][6] = hi.z; a[i][7] = hi.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* p = &Bs[st][16 * j + r16][8 * g];
      const float4 lo = *reinterpret_cast<const float4*>(p), hi = *reinterpret_cast<const float4*>(p + 4);
      b[j][0] = lo.x; b[j][1] = lo.y; b[j][2] = lo.z; b[j][3] = lo.w;
      b[j][4] = hi.x; b[j][5] = hi.y; b[j][6] = hi.z; b[j][7] = hi.w;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(a[i][q]), double(b[j][q]), acc[i][j], 0, 0, 0);
    if (c + 1 < nch) store(std::integral_constant<int, st ^ 1>{}, st ^ 1);   // the slot read in the previous chunk
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  load(kbeg, S0{});
  if (nch > 1) load(kbeg + GK, S1{});
  store(S0{}, 0);
  __syncthreads();
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    chunk(c, S0{});
    chunk(c + 1, S1{});
  }
  if (c < nch) chunk(c, S0{});
  // D[i][j]: lane holds column j = lane % 16, rows 4 * r + lane / 16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wave * 32 + i * 16 + r * 4 + g;
        const int e = e0 + j * 16 + r16;
        if (t < T && e < E) {
          if (partial) partial[(size_t(blockIdx.z) * T + t) * E + e] = acc[i][j][r];
          else logits[size_t(t) * E + e] = float(acc[i][j][r]);
        }
      }
}

// ---------------------------------------------------------------------------
// Router: one wavefront per token.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double score_d(double z, int func) {   // sigmoid or sqrt(softplus), in fp64
  const double ez = exp(-fabs(z));
  if (func == MOE_SCORE_SIGMOID) return z >= 0.0 ? 1.0 / (1.0 + ez) : ez / (1.0 + ez);
  return sqrt(fmax(z, 0.0) + log1p(ez));
}

__device__ __forceinline__ float score_fp64(float logit, int func) { return float(score_d(double(logit), func)); }

// The score and its slope f'(z) in fp32 arithmetic, each within a few units in the
// last place (one exp, one log1p or division, one sqrt, a rounding each).  Both
// functions increase, with f' <= 0.32 and |f''| < 0.1 everywhere (sigmoid:
// sigma (1 - sigma) and its derivative; sqrt(softplus): sigma / (2 f)).
__device__ __forceinline__ void score_slope_f32(float z, int func, float& s, float& slope) {
  const float ez = expf(-fabsf(z));
  const float sig = z >= 0.0f ? 1.0f / (1.0f + ez) : ez / (1.0f + ez);
  if (func == MOE_SCORE_SIGMOID) {
    s = sig;
    slope = sig * (1.0f - sig);
  } else {
    s = sqrtf(fmaxf(z, 0.0f) + log1pf(ez));
    slope = s > 0.0f ? sig / (2.0f * s) : 0.32f;
    slope = slope < 0.32f ? slope : 0.32f;           // (also when the quotient is not finite)
  }
}

constexpr int RT_WAVES = 4;
constexpr int RT_MAXE = 1024;
constexpr int RT_SLOTS = RT_MAXE / kWave;

__global__ __launch_bounds__(256) void router_kernel(const float* __restrict__ logits, const double* __restrict__ partial,
                                                     int nsplit, const float* __restrict__ bias,
                                                     int T, int E, int k, int n_group, int topk_group, int func,
                                                     int norm, float scale, int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_w) {
  __shared__ float s_lds[RT_WAVES][RT_MAXE];
  __shared__ float key_lds[RT_WAVES][RT_MAXE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * RT_WAVES + wave;
  const bool valid = t < T;                            // wave-uniform
  float* S = s_lds[wave];
  float* K = key_lds[wave];
  const float* lg = logits + size_t(valid ? t : 0) * E;
  for (int e = lane; e < E && valid; e += kWave) {
    float logit;
    if (partial) {                                      // K-split gate: fixed-order fp64 sum, one rounding
      double z = 0.0;
      const double* pp = partial + size_t(t) * E + e;
      const size_t ps = size_t(T) * E;
      int q = 0;
      for (; q + 8 <= nsplit; q += 8) {                 // 8 loads in flight, then the in-order sum
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pp[(q + u) * ps];
#pragma unroll
        for (int u = 0; u < 8; ++u) z += v[u];
      }
      for (; q < nsplit; ++q) z += pp[q * ps];
      logit = float(z);
    } else {
      logit = lg[e];
    }
    const float s = score_fp64(logit, func);
    float key = s + bias[e];
    key = (key == 0.0f) ? 0.0f : key;                  // -0 -> +0
    key = (key != key) ? -INFINITY : key;              // NaN ranks lowest
    S[e] = s;
    K[e] = key;
  }
  __syncthreads();
  if (!valid) return;

  // group selection: lane g scores group g by the sum of its two largest keys
  uint64_t kept_groups = ~0ull;
  const int gsz = E / n_group;
  if (n_group > 1) {
    uint64_t comp = 0;
    if (lane < n_group) {
      float top1 = -INFINITY, top2 = -INFINITY;
      for (int q = 0; q < gsz; ++q) {
        const float v = K[lane * gsz + q];
        if (v > top1) {
          top2 = top1;
          top1 = v;
        } else if (v > top2) {
          top2 = v;
        }
      }
      const float gscore = top1 + top2;
      comp = (uint64_t(orderable_f32(gscore)) << 32) | uint32_t(0xffffffffu - uint32_t(lane));
    }
    kept_groups = 0;
    for (int q = 0; q < topk_group; ++q) {
      const uint64_t best = wave_max_u64(comp);
      const int g = int(0xffffffffu - uint32_t(best));
      kept_groups |= 1ull << g;
      if (lane == g) comp = 0;
    }
  }

  // candidates held by this lane: experts lane + 64 * i
  uint64_t cand[RT_SLOTS];
#pragma unroll
  for (int i = 0; i < RT_SLOTS; ++i) {
    const int e = lane + i * kWave;
    uint64_t c = 0;
    if (e < E) {
      const int g = e / gsz;
      if ((kept_groups >> g) & 1ull) c = (uint64_t(orderable_f32(K[e])) << 32) | uint32_t(0xffffffffu - uint32_t(e));
    }
    cand[i] = c;
  }
  int my_pick = -1;                                      // lane j keeps the j-th pick
  for (int j = 0; j < k; ++j) {
    uint64_t loc = 0;
#pragma unroll
    for (int i = 0; i < RT_SLOTS; ++i) loc = cand[i] > loc ? cand[i] : loc;
    const uint64_t best = wave_max_u64(loc);
    const int e = int(0xffffffffu - uint32_t(best));
    if ((e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < RT_SLOTS; ++i)
        if (i == (e >> 6)) cand[i] = 0;
    }
    if (lane == j) my_pick = e;
  }
  // weights from the unbiased scores, normalised in fp64
  double sj = (lane < k) ? double(S[my_pick]) : 0.0;
  double sum = sj;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    const double w = norm ? sj / sum * double(scale) : sj * double(scale);
    topk_idx[size_t(t) * k + lane] = my_pick;
    topk_w[size_t(t) * k + lane] = float(w);
  }
}

// ---------------------------------------------------------------------------
// Gate at the bf16 MFMA rate with the same exact result (bf16 activations): a
// screen of the logits on the bf16 MFMA pipe, then an fp64 recompute of only the
// logits the selection can depend on.
//
// Screen: each fp32 gate weight is split, rounding to nearest, into two bf16 pieces
// and a remainder, w = w1 + w2 + w3 exactly with |w3| <= 2^-16 |w|; the products
// x * w1 and x * w2 are exact in fp32.  MFMAs add them in fp32, 256 products (4
// chunks of 32 K, both pieces) per chained accumulator, which is then added into an
// fp32 running total; the router adds the K splits' totals in fp64.  Whatever order
// the hardware adds in, an n-term fp32 sum is within gamma_n = n u / (1 - n u)
// (u = 2^-24) times the sum of |terms| of the exact one, so with G accumulator
// groups per split and by Cauchy-Schwarz the screened logit is within
//   eps = gamma_(256 + G + 2) |x|_2 (|w1|_2 + |w2|_2) + |x|_2 |w3|_2 + tiny
// of the exact dot product (tiny covers flushed subnormal inputs, products and
// partial sums).  The router turns that into an interval for each expert's
// selection key and recomputes exactly (fp64, one rounding to fp32, as the fp64
// gate does) every expert whose rank the intervals leave open: whether it is among
// the top k (and its group among the kept groups), or its order against another
// pick.  Selection and order are therefore those of the exact logits.  A pick whose
// rank was never in doubt keeps its screened score for the weight: the screen is an
// fp32-accumulated dot product of exact products, and its score is within
// lip * (eps + ulp) + ulp of the exact one (lip = 1/4 for sigmoid, < 0.32 for
// sqrt(softplus)).
// ---------------------------------------------------------------------------
constexpr int SCT = 256, SCE = 128, SK = 32, SGRP = 4;
constexpr int SC_WAVES = SCT / 32;                 // (SCT / 64) x 2 waves of 64 x 64

__device__ __forceinline__ uint32_t bf16_rn(float f) {   // round to nearest even; inf / nan stay inf / nan
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Pieces w1, w2 of every gate weight ([E][H] bf16 each) and per expert
// wn[4e..4e+2] = |w1|_2 + |w2|_2, |w3|_2, |w|_2, each rounded up (one 256-thread block
// per expert; fp64 sums of squares).
__global__ __launch_bounds__(256) void gate_prep(const float* __restrict__ wg, int E, int H, uint16_t* __restrict__ w1,
                                                 uint16_t* __restrict__ w2, float* __restrict__ wn) {
  __shared__ double red[4][4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double s1 = 0.0, s2 = 0.0, s3 = 0.0, sw = 0.0;
  for (int h = 4 * tid; h < H; h += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(wg + size_t(e) * H + h);
    const float wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t p1[4], p2[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      p1[q] = bf16_rn(wv[q]);
      const float f1 = __uint_as_float(p1[q] << 16), r = wv[q] - f1;   // exact
      p2[q] = bf16_rn(r);
      const float f2 = __uint_as_float(p2[q] << 16), f3 = r - f2;       // exact
      s1 += double(f1) * f1;
      s2 += double(f2) * f2;
      s3 += double(f3) * f3;
      sw += double(wv[q]) * wv[q];
    }
    *reinterpret_cast<uint2*>(w1 + size_t(e) * H + h) = uint2{p1[0] | (p1[1] << 16), p1[2] | (p1[3] << 16)};
    *reinterpret_cast<uint2*>(w2 + size_t(e) * H + h) = uint2{p2[0] | (p2[1] << 16), p2[2] | (p2[3] << 16)};
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    s1 += __shfl_xor(s1, off, 64);
    s2 += __shfl_xor(s2, off, 64);
    s3 += __shfl_xor(s3, off, 64);
    sw += __shfl_xor(sw, off, 64);
  }
  if (lane == 0) {
    red[wave][0] = s1;
    red[wave][1] = s2;
    red[wave][2] = s3;
    red[wave][3] = sw;
  }
  __syncthreads();
  if (tid == 0) {
    s1 = red[0][0] + red[1][0] + red[2][0] + red[3][0];
    s2 = red[0][1] + red[1][1] + red[2][1] + red[3][1];
    s3 = red[0][2] + red[1][2] + red[2][2] + red[3][2];
    sw = red[0][3] + red[1][3] + red[2][3] + red[3][3];
    constexpr double up = 1.0 + 0x1p-20;              // covers the fp64 sums and the rounding to fp32
    wn[4 * e + 0] = float((sqrt(s1) + sqrt(s2)) * up);
    wn[4 * e + 1] = float(sqrt(s3) * up);
    wn[4 * e + 2] = float(sqrt(sw) * up);
    wn[4 * e + 3] = 0.0f;
  }
}

typedef __attribute__((ext_vector_type(4))) float rf32x4;

// Screened logits: a 256-token x 128-expert tile per 512-thread block (one per CU),
// wave (wt, we) owning tokens 64 wt .. and experts 64 we .. (4 x 4 MFMA 16x16x32
// tiles).  K runs in chunks of 32 through a ring of SC_NS LDS stages filled by direct
// global -> LDS copies (16 bytes per lane, no registers), SC_NS - 1 chunks ahead of
// the one being multiplied.  A stage holds 256 x rows, then 128 w1 rows, then 128 w2
// rows of 64 bytes; the 16-byte segment s of row r sits in slot s ^ ((r >> 1) & 3): the MFMA
// operand reads (16 rows, one segment per 16 lanes) are then free of bank conflicts
// (measured: SQ_LDS_BANK_CONFLICT is zero for this pattern and 4 cycles per read
// for the unswizzled rows, for s ^ ((r >> 2) & 3) and for 80-byte padded rows).
// Blocks are dealt to the 8 XCDs in turn, so logical tile i*N/8 + j runs on XCD i:
// the expert tiles of one token tile, which read the same x rows, share an L2.
// part[split][t][e]: the split's fp32 total.  (Measured against 128 x 128 tiles,
// two per CU, with 3 stages: 0.052 / 0.093 / 0.17 ms against 0.070 / 0.106 / 0.19 ms
// for 8192 x 256, 4096 x 896 and 16384 x 384 at H = 7168.)
constexpr int SC_NS = 4;
constexpr int SC_STAGE = (SCT + 2 * SCE) * SK * 2;   // 32 KiB
constexpr int SC_CPW = (SCT + 2 * SCE) / 16 / SC_WAVES;   // 16-row copies per wave and chunk

typedef __attribute__((address_space(3))) void* sc_lds_ptr_t;

__device__ __forceinline__ int sc_swz(int r, int seg) { return r * 64 + ((seg ^ ((r >> 1) & 3)) << 4); }

__device__ __forceinline__ void sc_copy16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (sc_lds_ptr_t)lds, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void sc_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

__global__ __launch_bounds__(SCT * 2, 1) void gate_screen(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w2,
    float* __restrict__ part, float* __restrict__ xsq, int T, int E, int H, int kchunk, int e_tiles, int tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[SC_NS][SC_STAGE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4, wt = wave >> 1, we = wave & 1;
  const int nb = gridDim.x, b = blockIdx.x;
  const int lg = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  const int split = lg / tiles, rest = lg % tiles;
  const int t0 = (rest / e_tiles) * SCT, e0 = (rest % e_tiles) * SCE;
  const int kbeg = split * kchunk, nch = kchunk / SK;
  // copies of one chunk: wave w fills 16-row blocks SC_CPW w .. of the stage (x rows,
  // then w1, then w2); lane l takes row l >> 2 of the block and the segment stored in
  // its slot l & 3.  Rows past T / E read the last row (their results are dropped).
  const int lr = lane >> 2, lseg = (lane & 3) ^ ((lane >> 3) & 3);
  const char* src[SC_CPW];
  int dst[SC_CPW];
#pragma unroll
  for (int i = 0; i < SC_CPW; ++i) {
    const int blk = wave * SC_CPW + i;
    if (blk < SCT / 16) {
      src[i] = reinterpret_cast<const char*>(x + size_t(min(t0 + 16 * blk + lr, T - 1)) * H + kbeg) + lseg * 16;
    } else {
      const int bb = blk - SCT / 16, r = 16 * (bb % (SCE / 16)) + lr;
      const uint16_t* w = bb < SCE / 16 ? w1 : w2;
      src[i] = reinterpret_cast<const char*>(w + size_t(min(e0 + r, E - 1)) * H + kbeg) + lseg * 16;
    }
    dst[i] = blk * 1024;
  }
  auto issue = [&](int c, int slot) {
#pragma unroll
    for (int j = 0; j < SC_CPW; ++j) sc_copy16(src[j] + c * 64, &ring[slot][0] + dst[j]);
  };
  rf32x4 cur[4][4], tot[4][4];
  const rf32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  // the first expert tile's token waves also sum the squares of their x rows (exact
  // products, fp32 sums of positive terms) for the router's error bound
  const bool do_sq = (rest % e_tiles) == 0 && we == 0;
  float sq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cur[i][j] = z4;
      tot[i][j] = z4;
    }
  // Every iteration issues one chunk's copies (past the end: chunk nch-1 again, into
  // a slot no later iteration reads), so the count of this wave's copies newer than
  // chunk c's is always SC_CPW (SC_NS - 2).
#pragma unroll
  for (int c = 0; c < SC_NS - 1; ++c) issue(min(c, nch - 1), c);
  for (int c = 0; c < nch; ++c) {
    sc_wait_vmcnt<SC_CPW * (SC_NS - 2)>();
    // every wave's copies of chunk c are in LDS, and every wave is done with slot
    // (c - 1) % SC_NS, which the next copies fill
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue(min(c + SC_NS - 1, nch - 1), (c + SC_NS - 1) % SC_NS);
    const uint8_t* st = ring[c % SC_NS];
    bf16x8 a[4], bw[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(st + sc_swz(wt * 64 + 16 * i + r16, g));
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bw[p][j] = *reinterpret_cast<const bf16x8*>(st + (SCT + p * SCE) * 64 + sc_swz(we * 64 + 16 * j + r16, g));
    if (do_sq) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = __builtin_bit_cast(uint4, a[i]);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(w4[q] << 16), hi = __uint_as_float(w4[q] & 0xffff0000u);
          sq[i] = fmaf(lo, lo, sq[i]);
          sq[i] = fmaf(hi, hi, sq[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cur[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[1][j], a[i], cur[i][j], 0, 0, 0);
        cur[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[0][j], a[i], cur[i][j], 0, 0, 0);
      }
    if ((c % SGRP) == SGRP - 1 || c + 1 == nch) {   // close the accumulator group
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tot[i][j] += cur[i][j];
          cur[i][j] = z4;
        }
    }
  }
  sc_wait_vmcnt<0>();                                // no copy into LDS outlives the block
  if (do_sq) {                                       // lanes r16 + 16 g hold row r16's four K slices
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sq[i] += __shfl_xor(sq[i], 16, 64);
      sq[i] += __shfl_xor(sq[i], 32, 64);
      const int t = t0 + wt * 64 + 16 * i + r16;
      if (g == 0 && t < T) xsq[size_t(split) * T + t] = sq[i];
    }
  }
  // D lane l, register r: expert row 4(l >> 4) + r of the 16-expert block, token l & 15
  float* out = part + size_t(split) * T * E;
  const bool vec = (E & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + wt * 64 + 16 * i + r16;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + we * 64 + 16 * j + 4 * g;
      float* o = out + size_t(t) * E + e;
      if (vec && e + 3 < E) {
        *reinterpret_cast<float4*>(o) = make_float4(tot[i][j][0], tot[i][j][1], tot[i][j][2], tot[i][j][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e + r < E) o[r] = tot[i][j][r];
      }
    }
  }
}

__device__ __forceinline__ float ulp32(float v) {   // spacing of fp32 values at |v| (>= the least normal's)
  const uint32_t ex = (__float_as_uint(v) >> 23) & 0xffu;
  return __uint_as_float((ex > 23u ? ex - 23u : 1u) << 23);
}

__device__ __forceinline__ float selection_key(float s, float b) {
  float key = s + b;
  key = (key == 0.0f) ? 0.0f : key;                 // -0 -> +0
  return (key != key) ? -INFINITY : key;            // NaN ranks lowest
}

__device__ __forceinline__ float from_orderable(uint64_t c) {   // value of a (orderable << 32 | ~e) key
  const uint32_t o = uint32_t(c >> 32);
  return __uint_as_float((o >> 31) ? o & 0x7fffffffu : ~o);
}

// Largest value (and its expert, ties to the lower index) among `vals` over experts
// that `want` selects, as the u64 (orderable value << 32 | ~e).
template <typename Pred>
__device__ __forceinline__ uint64_t wave_best(const float* vals, int E, int lane, Pred want) {
  uint64_t loc = 0;
  for (int e = lane; e < E; e += kWave)
    if (want(e)) {
      const uint64_t c = (uint64_t(orderable_f32(vals[e])) << 32) | uint32_t(0xffffffffu - uint32_t(e));
      loc = c > loc ? c : loc;
    }
  return wave_max_u64(loc);
}

constexpr int RS_WAVES = 4;
constexpr int RS_FLOATS_PER_EXPERT = 5;            // LO, HI, exact key, exact score, state

// One wavefront per token.
__global__ __launch_bounds__(256, 2) void router_screen_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ wn,
    const float* __restrict__ part, const float* __restrict__ xsq, int nsplit, const float* __restrict__ bias, int T,
    int E, int H, int k,
    int n_group, int topk_group, int func, int norm, float scale, double gam, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  extern __shared__ float rs_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * RS_WAVES + wave;
  if (t >= T) return;                                 // no block-wide barrier below
  float* LO = rs_lds + size_t(wave) * RS_FLOATS_PER_EXPERT * E;
  float *HI = LO + E, *KX = HI + E, *SX = KX + E;
  uint32_t* ST = reinterpret_cast<uint32_t*>(SX + E);   // 1: exact; 2: recompute requested; 4: candidate; 8: kept
  int* CL = reinterpret_cast<int*>(rs_lds + size_t(RS_WAVES) * RS_FLOATS_PER_EXPERT * E) + wave * kWave;
  // the row (buffer range check: lanes past its end read zeros), and |x_t|_2 from the
  // screen's sums of squares.  Each is an fp32 sum of at most H/4 + 2 exact positive
  // terms, so at most a factor 1 - gamma_(H/4+2) below the exact one: times
  // 1 + H 2^-22 covers that with room; 2^-50 covers squares flushed as subnormals.
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + size_t(t) * H), short(0), H * 2, 0x00020000);
  double xs = 0.0;
  for (int q = 0; q < nsplit; ++q) xs += double(xsq[size_t(q) * T + t]);
  const double xnorm = sqrt(xs * (1.0 + double(H) * 0x1p-22)) * (1.0 + 0x1p-20) + 0x1p-50;
  const double sub = 0x1p-118 * sqrt(double(H));     // flushed subnormal inputs: 2^-126 per |other factor|, ...
  // exact logit of expert e: fp64 products (exact) and fp64 sums in a fixed order,
  // one rounding to fp32.  The row and the gate row stream together in passes of
  // 2048 (8 loads of each per lane in flight); loads past the end return zeros.
  auto exact = [&](int e) -> float {
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(wg + size_t(e) * H), short(0), H * 4, 0x00020000);
    double s0 = 0.0, s1 = 0.0;
    for (int h0 = 0; h0 < H; h0 += 2048) {
      uint2 xq[8];
      float4 wv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int h = h0 + 4 * lane + 256 * i;
        xq[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rx, 2 * h, 0, 0));
        wv[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rw, 4 * h, 0, 0));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s0 = fma(double(__uint_as_float(xq[i].x << 16)), double(wv[i].x), s0);
        s1 = fma(double(__uint_as_float(xq[i].x & 0xffff0000u)), double(wv[i].y), s1);
        s0 = fma(double(__uint_as_float(xq[i].y << 16)), double(wv[i].z), s0);
        s1 = fma(double(__uint_as_float(xq[i].y & 0xffff0000u)), double(wv[i].w), s1);
      }
    }
    double s = s0 + s1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    return float(s);
  };
  // screened keys -> intervals [LO, HI] that hold the exact keys
  for (int e = lane; e < E; e += kWave) {
    double zs = 0.0;
    for (int q = 0; q < nsplit; ++q) zs += double(part[(size_t(q) * T + t) * E + e]);
    const float l32 = float(zs);
    const float4 n = *reinterpret_cast<const float4*>(wn + 4 * e);
    const double eps = gam * xnorm * double(n.x) + xnorm * double(n.y) + sub * (xnorm + double(n.z)) + 0x1p-100;
    // The exact fp32 logit is within dl of l32 (twice the bound, for whatever rounding
    // the MFMA sums use, and two fp32 roundings).  By the mean value theorem (twice)
    // the exact score is then within (f'(l32) + 0.125 dl) dl of f(l32); the fp32
    // evaluation adds at most 2^-16 relative (far more than its error) and the
    // rounding of the exact score one unit.  The exact key, an fp32 sum with the
    // bias, lies between the same sums of the score interval's ends.
    const double dl = 2.0 * eps + 2.0 * double(ulp32(l32));
    float sc, slope;
    score_slope_f32(l32, func, sc, slope);
    const float hw = float((double(slope) * (1.0 + 0x1p-10) + 0.125 * dl) * dl) + sc * 0x1p-16f + ulp32(sc);
    const float u = ulp32(fmaxf(sc, hw));
    const float klo = ((sc - hw) - u) + bias[e], khi = ((sc + hw) + u) + bias[e];
    const float lo = klo - ulp32(klo), hi = khi + ulp32(khi);
    if (!(dl < INFINITY) || !(fabs(zs) < INFINITY) || !(lo > -INFINITY) || !(hi == hi) || hi == INFINITY) {
      LO[e] = -INFINITY;                             // NaN, infinity or overflow: recompute
      HI[e] = INFINITY;
    } else {
      LO[e] = lo;
      HI[e] = hi;
    }
    SX[e] = l32;                                     // the screened logit (its score: when listed)
    ST[e] = 0u;
  }
  auto recompute = [&]() {                           // exact keys of the requested experts
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      uint64_t m = __ballot(e < E && (ST[e] & 2u));
      while (m) {
        const int q = __builtin_ctzll(m);
        m &= m - 1;
        const int ee = base + q;
        const float l = exact(ee);
        if (lane == 0) {
          const float s = score_fp64(l, func);
          SX[ee] = s;
          KX[ee] = selection_key(s, bias[ee]);
          ST[ee] = (ST[ee] & ~2u) | 1u;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  // ---- groups: keep topk_group by the sum of each group's two largest keys
  uint64_t kept = ~0ull;
  const int gsz = E / n_group;
  if (n_group > 1) {
    // lane g < n_group: bounds of group g's score
    float glo = -INFINITY, ghi = -INFINITY;
    if (lane < n_group) {
      float l1 = -INFINITY, l2 = -INFINITY, h1 = -INFINITY, h2 = -INFINITY;
      for (int q = 0; q < gsz; ++q) {
        const int e = lane * gsz + q;
        const float a = LO[e], b = HI[e];
        if (a > l1) { l2 = l1; l1 = a; } else if (a > l2) l2 = a;
        if (b > h1) { h2 = h1; h1 = b; } else if (b > h2) h2 = b;
      }
      const float sl = l1 + l2, sh = h1 + h2;
      glo = sl - 2.0f * ulp32(sl);
      ghi = sh + 2.0f * ulp32(sh);
    }
    // the topk_group-th largest lower end, the (topk_group+1)-th largest upper end
    auto kth = [&](float v, int kk) {                 // kk-th largest of lanes' v (lanes < n_group)
      uint64_t c = lane < n_group ? ((uint64_t(orderable_f32(v)) << 32) | uint32_t(0xffffffffu - uint32_t(lane))) : 0;
      uint64_t best = 0;
      for (int q = 0; q < kk; ++q) {
        best = wave_max_u64(c);
        if (lane == int(0xffffffffu - uint32_t(best))) c = 0;
      }
      return best;
    };
    const float Lg = from_orderable(kth(glo, topk_group));
    const float Hg = topk_group < n_group ? from_orderable(kth(ghi, topk_group + 1)) : -INFINITY;
    const bool in_for_sure = lane < n_group && glo > Hg;
    const bool out_for_sure = lane < n_group && ghi < Lg;
    const uint64_t sure_in = __ballot(in_for_sure), amb = __ballot(lane < n_group && !in_for_sure && !out_for_sure);
    kept = sure_in;
    const int slots = topk_group - __popcll(sure_in);
    if (slots > 0) {
      // exact scores of the ambiguous groups: recompute every member that may be
      // among the group's two largest keys
      for (int gq = 0; gq < n_group; ++gq) {
        if (!((amb >> gq) & 1ull)) continue;
        float l1 = -INFINITY, l2 = -INFINITY;
        for (int q = lane; q < gsz; q += kWave) {
          const float a = LO[gq * gsz + q];
          if (a > l1) { l2 = l1; l1 = a; } else if (a > l2) l2 = a;
        }
        // second largest lower end of the group over the wave
        for (int off = 32; off >= 1; off >>= 1) {
          const float o1 = __shfl_xor(l1, off, 64), o2 = __shfl_xor(l2, off, 64);
          const float n1 = fmaxf(l1, o1);
          const float n2 = fmaxf(fminf(l1, o1), fmaxf(l2, o2));
          l1 = n1;
          l2 = n2;
        }
        for (int q = lane; q < gsz; q += kWave) {
          const int e = gq * gsz + q;
          if (HI[e] >= l2 && !(ST[e] & 1u)) ST[e] |= 2u;
        }
      }
      __builtin_amdgcn_wave_barrier();
      recompute();
      // exact group scores, then the best `slots` ambiguous groups (ties: lower group)
      uint64_t c = 0;
      if ((amb >> lane) & 1ull && lane < n_group) {
        float k1 = -INFINITY, k2 = -INFINITY;
        for (int q = 0; q < gsz; ++q) {
          const int e = lane * gsz + q;
          if (!(ST[e] & 1u)) continue;              // not among the group's two largest
          const float v = KX[e];
          if (v > k1) { k2 = k1; k1 = v; } else if (v > k2) k2 = v;
        }
        c = (uint64_t(orderable_f32(k1 + k2)) << 32) | uint32_t(0xffffffffu - uint32_t(lane));
      }
      for (int q = 0; q < slots; ++q) {
        const uint64_t best = wave_max_u64(c);
        const int gb = int(0xffffffffu - uint32_t(best));
        kept |= 1ull << gb;
        if (lane == gb) c = 0;
      }
    }
  }
  // ---- kept experts: state bit 8
  for (int e = lane; e < E; e += kWave)
    if (n_group == 1 || ((kept >> (e / gsz)) & 1ull)) ST[e] |= 8u;
  __builtin_amdgcn_wave_barrier();
  // ---- candidates: kept experts whose upper end reaches the k-th largest lower end
  // L (every other expert has k kept experts surely above it).  The k-th largest of
  // the lanes' own largest lower ends is at most L: the experts above that bound are
  // listed first, and L is then found among them.  (If more than 64 pass the bound,
  // L comes from k rounds over every expert.)
  auto compact = [&](float thr) {                    // candidates HI >= thr, the first 64 listed in CL
    int n = 0;
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const bool cand = e < E && (ST[e] & 8u) && HI[e] >= thr;
      const uint64_t m = __ballot(cand);
      if (e < E) ST[e] = (ST[e] & ~4u) | (cand ? 4u : 0u);
      if (cand) {
        const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
        if (pos < kWave) CL[pos] = e;
      }
      n += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    return n;
  };
  float lane_max = -INFINITY;
  for (int e = lane; e < E; e += kWave)
    if (ST[e] & 8u) lane_max = fmaxf(lane_max, LO[e]);
  uint64_t lb = (uint64_t(orderable_f32(lane_max)) << 32) | uint32_t(0xffffffffu - uint32_t(lane));
  uint64_t lk = 0;
  for (int q = 0; q < k; ++q) {
    lk = wave_max_u64(lb);
    if (lane == int(0xffffffffu - uint32_t(lk))) lb = 0;
  }
  int nc = compact(from_orderable(lk));
  bool l_known = false;                              // L applied to the list yet?
  if (nc > kWave) {
    for (int e = lane; e < E; e += kWave) ST[e] &= ~4u;
    __builtin_amdgcn_wave_barrier();
    for (int q = 0; q < k; ++q) {
      lk = wave_best(LO, E, lane, [&](int e) { return (ST[e] & 12u) == 8u; });
      const int e = int(0xffffffffu - uint32_t(lk));
      if (lane == 0) ST[e] |= 4u;                    // (temporarily marks the k largest lower ends)
      __builtin_amdgcn_wave_barrier();
    }
    nc = compact(from_orderable(lk));
    l_known = true;
  }
  int my_pick = -1;
  if (nc <= kWave) {
    // Candidate c on lane c, with its key interval (a point once exact).  It is out
    // for sure when k others lie entirely above it.  An expert that is not out and
    // whose interval meets another such candidate's gets its exact key; every other
    // one is ordered correctly against all the rest by its screened key, and keeps
    // its screened score for the weight.
    bool has = lane < nc;
    const int ce = has ? CL[lane] : 0;
    if (!l_known) {                                  // L among the listed lower ends
      uint64_t c = has ? ((uint64_t(orderable_f32(LO[ce])) << 32) | uint32_t(0xffffffffu - uint32_t(ce))) : 0;
      uint64_t best = 0;
      for (int q = 0; q < k; ++q) {
        best = wave_max_u64(c);
        if (has && int(0xffffffffu - uint32_t(best)) == ce) c = 0;
      }
      has = has && HI[ce] >= from_orderable(best);
    }
    const bool ex = has && (ST[ce] & 1u);
    if (has && !ex) {                                // screened score and key (inside [LO, HI])
      const float sc = score_fp64(SX[ce], func);
      SX[ce] = sc;
      KX[ce] = selection_key(sc, bias[ce]);
    }
    const float lo = has ? (ex ? KX[ce] : LO[ce]) : -INFINITY;   // lanes without a candidate: never above,
    const float hi = has ? (ex ? KX[ce] : HI[ce]) : -INFINITY;   // and out
    int above = 0;
    for (int d = 0; d < nc; ++d) above += (__shfl(lo, d, 64) > hi) ? 1 : 0;
    const bool out = !has || above >= k;
    bool meets = false;
    for (int d = 0; d < nc; ++d) {
      const float lod = __shfl(lo, d, 64), hid = __shfl(hi, d, 64);
      const bool outd = __shfl(int(out), d, 64) != 0;
      meets = meets || (d != lane && !outd && hid >= lo && lod <= hi);
    }
    if (has && !out && meets && !ex) ST[ce] |= 2u;
    __builtin_amdgcn_wave_barrier();
    recompute();
    // the k best candidates that are not out, by key, ties to the lower index
    uint64_t c = (has && !out) ? ((uint64_t(orderable_f32(KX[ce])) << 32) | uint32_t(0xffffffffu - uint32_t(ce))) : 0;
    for (int j = 0; j < k; ++j) {
      const uint64_t best = wave_max_u64(c);
      const int e = int(0xffffffffu - uint32_t(best));
      if (has && e == ce) c = 0;
      if (lane == j) my_pick = e;
    }
  } else {
    // many near-equal keys: exact keys for every candidate, then the k best
    for (int e = lane; e < E; e += kWave)
      if ((ST[e] & 4u) && !(ST[e] & 1u)) ST[e] |= 2u;
    __builtin_amdgcn_wave_barrier();
    recompute();
    for (int j = 0; j < k; ++j) {
      const uint64_t best = wave_best(KX, E, lane, [&](int e) { return (ST[e] & 4u) != 0; });
      const int e = int(0xffffffffu - uint32_t(best));
      if (lane == 0) ST[e] &= ~4u;
      __builtin_amdgcn_wave_barrier();
      if (lane == j) my_pick = e;
    }
  }
  double sj = (lane < k) ? double(SX[my_pick]) : 0.0;
  double sum = sj;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    const double w = norm ? sj / sum * double(scale) : sj * double(scale);
    topk_idx[size_t(t) * k + lane] = my_pick;
    topk_w[size_t(t) * k + lane] = float(w);
  }
}

// ---------------------------------------------------------------------------
// Which gate runs, and how it is split over K.
// ---------------------------------------------------------------------------
// The screen needs bf16 activations; below a few hundred tokens the fp64 gate is as
// fast.
static bool use_screen(const moe_config_t& c) {
  return c.recipe != MOE_RECIPE_F32 && c.hidden % SK == 0 && c.num_tokens >= 512;
}

// fp64 gate: the d (a divisor of the K chunks, <= 32) with the least estimated
// time.  The kernel is fp64-MFMA bound and two 128 x 64 blocks share a CU (LDS), so
// a CU that holds L blocks takes L times as long as one block alone would with a
// second one beside it, and a lone block leaves half its CU's issue slots unused:
// time ~ (max(L, 2) + 1/2) * (K/d chunks), L = ceil(blocks / 256), the half block
// for the uneven finish of the last ones.  Every split beyond the first adds a
// T x E fp64 partial written once and read once.  Per-chunk time and bandwidth are
// round measured figures.
static int gate_ksplit_f64(const moe_config_t& c) {
  const int tiles = ((c.num_experts + GE - 1) / GE) * ((c.num_tokens + GT - 1) / GT);
  const int steps = c.hidden / GK;
  constexpr double chunk_s = 1.7e-6, bytes_per_s = 5e12;
  int best = 1;
  double best_t = 0.0;
  for (int d = 1; d <= steps && d <= 32; ++d) {
    if (steps % d) continue;
    const int64_t per_cu = (int64_t(tiles) * d + 255) / 256;
    const double t = (double(std::max<int64_t>(per_cu, 2)) + 0.5) * (steps / d) * chunk_s +
                     (d > 1 ? double(d) * c.num_tokens * c.num_experts * 16.0 / bytes_per_s : 0.0);
    if (d == 1 || t < 0.97 * best_t) {             // a split must win clearly
      best = d;
      best_t = t;
    }
  }
  return best;
}

// Screen: one 256 x 128 block per CU, about 0.93 us per 32-deep chunk (measured), so
// time ~ ceil(blocks / 256) * (K/d chunks) * t_chunk; every split beyond the first
// adds a T x E fp32 partial written and read once.  Splits keep >= 8 chunks each.
static int gate_ksplit_screen(const moe_config_t& c) {
  const int64_t tiles = int64_t((c.num_experts + SCE - 1) / SCE) * ((c.num_tokens + SCT - 1) / SCT);
  const int steps = c.hidden / SK;
  constexpr double chunk_s = 0.93e-6, bytes_per_s = 5e12;
  int best = 1;
  double best_t = 0.0;
  for (int d = 1; d <= 32 && d <= steps; ++d) {
    if (steps % d || (d > 1 && steps / d < 8)) continue;
    const int64_t per_cu = (tiles * d + 255) / 256;
    const double t = double(per_cu) * (steps / d) * chunk_s +
                     double(d - 1) * c.num_tokens * c.num_experts * 8.0 / bytes_per_s;
    if (d == 1 || t < 0.97 * best_t) {
      best = d;
      best_t = t;
    }
  }
  return best;
}

namespace {
struct RouteWs {                                     // byte offsets in the route workspace
  size_t logits, partial, part, xsq, w1, w2, wn, total;
};
RouteWs route_ws(const moe_config_t& c) {
  RouteWs r{};
  const size_t T = size_t(c.num_tokens), E = size_t(c.num_experts), H = size_t(c.hidden);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += (bytes + 255) & ~size_t(255); return at; };
  if (use_screen(c)) {
    const int ks = gate_ksplit_screen(c);
    r.part = take(size_t(ks) * T * E * 4);
    r.xsq = take(size_t(ks) * T * 4);
    r.w1 = take(E * H * 2);
    r.w2 = take(E * H * 2);
    r.wn = take(E * 16);
  } else {
    const int ks = gate_ksplit_f64(c);
    r.logits = take(T * E * 4);
    r.partial = take(ks > 1 ? size_t(ks) * T * E * 8 : 0);
  }
  r.total = o;
  return r;
}
}  // namespace

size_t route_workspace_bytes(const moe_config_t& c) { return route_ws(c).total; }

static void launch_router_screen(const moe_config_t& c, const uint16_t* xb, const float* gate_w, const float* wn,
                                 const float* part, const float* xsq, int ks, const float* bias, double gam,
                                 int32_t* topk_idx, float* topk_w, hipStream_t st) {
  const int T = c.num_tokens, E = c.num_experts;
  const size_t lds = (size_t(RS_WAVES) * RS_FLOATS_PER_EXPERT * E + RS_WAVES * kWave) * 4;   // <= 81 KiB
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&router_screen_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  router_screen_kernel<<<(T + RS_WAVES - 1) / RS_WAVES, 256, lds, st>>>(
      xb, gate_w, wn, part, xsq, ks, bias, T, E, c.hidden, c.top_k, c.n_group, c.topk_group, c.score_func,
      c.norm_topk_prob, c.routed_scaling_factor, gam, topk_idx, topk_w);
}

hipError_t launch_route(const moe_config_t& c, const void* x, const float* gate_w, const float* bias,
                        int32_t* topk_idx, float* topk_w, void* ws, hipStream_t st) {
  const int T = c.num_tokens, E = c.num_experts, H = c.hidden;
  const RouteWs r = route_ws(c);
  char* base = static_cast<char*>(ws);
  if (!use_screen(c)) {                              // the fp64 gate
    const int ks = gate_ksplit_f64(c);
    float* logits = reinterpret_cast<float*>(base + r.logits);
    double* partial = ks > 1 ? reinterpret_cast<double*>(base + r.partial) : nullptr;
    dim3 gg((E + GE - 1) / GE, (T + GT - 1) / GT, ks);
    {
      ProfScope p(MOE_K_GATE, st);
      if (c.recipe == MOE_RECIPE_F32)
        gate_logits_f64<float><<<gg, 256, 0, st>>>(static_cast<const float*>(x), gate_w, logits, partial, T, E, H,
                                                    H / ks);
      else
        gate_logits_f64<uint16_t><<<gg, 256, 0, st>>>(static_cast<const uint16_t*>(x), gate_w, logits, partial, T,
                                                       E, H, H / ks);
    }
    ProfScope p(MOE_K_ROUTER, st);
    router_kernel<<<(T + RT_WAVES - 1) / RT_WAVES, 256, 0, st>>>(logits, partial, ks, bias, T, E, c.top_k,
                                                                c.n_group, c.topk_group, c.score_func,
                                                                c.norm_topk_prob, c.routed_scaling_factor, topk_idx,
                                                                topk_w);
    return hipGetLastError();
  }
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const int ks = gate_ksplit_screen(c);
  float* part = reinterpret_cast<float*>(base + r.part);
  uint16_t* w1 = reinterpret_cast<uint16_t*>(base + r.w1);
  uint16_t* w2 = reinterpret_cast<uint16_t*>(base + r.w2);
  float* wn = reinterpret_cast<float*>(base + r.wn);
  float* xsq = reinterpret_cast<float*>(base + r.xsq);
  const int kchunk = H / ks, e_tiles = (E + SCE - 1) / SCE, tiles = e_tiles * ((T + SCT - 1) / SCT);
  {
    ProfScope p(MOE_K_GATE, st);
    gate_prep<<<E, 256, 0, st>>>(gate_w, E, H, w1, w2, wn);
    gate_screen<<<tiles * ks, SCT * 2, 0, st>>>(xb, w1, w2, part, xsq, T, E, H, kchunk, e_tiles, tiles);
  }
  // error bound factor: gamma_n with n = 256 (one accumulator group) + groups + 2
  const int groups = (kchunk / SK + SGRP - 1) / SGRP;
  const double n = double(2 * SK * SGRP + groups + 2), u = 0x1p-24;
  const double gam = n * u / (1.0 - n * u);
  ProfScope p(MOE_K_ROUTER, st);
  launch_router_screen(c, xb, gate_w, wn, part, xsq, ks, bias, gam, topk_idx, topk_w, st);
  return hipGetLastError();
}

}  // namespace moe
