// MoEGate.forward on gfx950: gate logits, scores, noaux_tc grouped top-k, weights.
//
// Walk-through of the DeepSeek-V3 architecture (pwwt.cn/news/5781524), section 3:
// 3.1 the gate matrix [E, H] times the hidden state in FP32, sigmoid per expert;
// 3.2 + e_score_correction_bias, group top-2 sums, keep topk_group groups, top-k;
// 3.3 normalise the k picked scores to sum 1, times routed_scaling_factor.
// sqrtsoftplus is the DeepSeek-V4-Pro score (lzwjava.github.io, architecture).
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
    if (c + 2 < nch) load(kbeg + (c + 2) * GK, setc);   // set st held chunk c, already in LDS
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
__device__ __forceinline__ float score_fp64(float logit, int func) {
  const double z = double(logit);
  const double ez = exp(-fabs(z));
  double s;
  if (func == MOE_SCORE_SIGMOID) {
    s = z >= 0.0 ? 1.0 / (1.0 + ez) : ez / (1.0 + ez);
  } else {
    s = sqrt(fmax(z, 0.0) + log1p(ez));
  }
  return float(s);
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
// K splits of the gate GEMM: the d (a divisor of the K chunks, <= 32) with the
// least estimated time.  The kernel is fp64-MFMA bound and two 128 x 64 blocks
// share a CU (LDS), so a CU that holds L blocks takes L times as long as one
// block alone would with a second one beside it, and a lone block leaves half its
// CU's issue slots unused: time ~ (max(L, 2) + 1/2) * (K/d chunks), L =
// ceil(blocks / 256), the half block for the uneven finish of the last ones.
// Every split beyond the first adds a T x E fp64 partial written once and read
// once.  Per-chunk time and bandwidth are round measured figures.
int gate_ksplit(const moe_config_t& c) {
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

hipError_t launch_route(const moe_config_t& c, const void* x, const float* gate_w, const float* bias,
                        int32_t* topk_idx, float* topk_w, float* logits_ws, double* partial_ws, hipStream_t st) {
  const int T = c.num_tokens, E = c.num_experts, H = c.hidden;
  const int ks = gate_ksplit(c);
  double* partial = ks > 1 ? partial_ws : nullptr;
  dim3 gg((E + GE - 1) / GE, (T + GT - 1) / GT, ks);
  {
    ProfScope p(MOE_K_GATE, st);
    if (c.recipe == MOE_RECIPE_F32)
      gate_logits_f64<float><<<gg, 256, 0, st>>>(static_cast<const float*>(x), gate_w, logits_ws, partial, T, E, H,
                                                  H / ks);
    else
      gate_logits_f64<uint16_t><<<gg, 256, 0, st>>>(static_cast<const uint16_t*>(x), gate_w, logits_ws, partial, T,
                                                     E, H, H / ks);
  }
  ProfScope p(MOE_K_ROUTER, st);
  router_kernel<<<(T + RT_WAVES - 1) / RT_WAVES, 256, 0, st>>>(logits_ws, partial, ks, bias, T, E, c.top_k, c.n_group,
                                                              c.topk_group, c.score_func, c.norm_topk_prob,
                                                              c.routed_scaling_factor, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
