// MoEGate.forward on gfx950: gate logits, scores, noaux_tc grouped top-k, weights.
//
// Walk-through of the DeepSeek-V3 architecture (pwwt.cn/news/5781524), section 3:
// 3.1 the gate matrix [E, H] times the hidden state in FP32, sigmoid per expert;
// 3.2 + e_score_correction_bias, group top-2 sums, keep topk_group groups, top-k;
// 3.3 normalise the k picked scores to sum 1, times routed_scaling_factor.
// sqrtsoftplus is the DeepSeek-V4-Pro score (lzwjava.github.io, architecture).
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Gate logits: logits[t][e] = fp32( sum_h x[t][h] * Wg[e][h] ), accumulated in fp64.
// Products of bf16/fp32 by fp32 values are exact in fp64, so the only rounding
// that matters is the final one to fp32: the kernel reproduces the correctly
// rounded FP32 linear layer except when the fp64 sum lands within ~1e-16
// (relative) of an fp32 rounding boundary.
//
// fp64 MFMA 16x16x4: a 64x64 (token x expert) tile per 256-thread block; each
// wave owns a 32x32 quarter = 2x2 MFMA tiles.  K is staged through LDS in
// chunks of 32, converted to fp64 once on the way in.
// ---------------------------------------------------------------------------
constexpr int GT = 64, GE = 64, GK = 32, GPAD = GK + 1;

template <typename XT>
__device__ __forceinline__ double load_x64(const XT* p);
template <>
__device__ __forceinline__ double load_x64<float>(const float* p) { return double(*p); }
template <>
__device__ __forceinline__ double load_x64<uint16_t>(const uint16_t* p) { return double(bf16_to_f32(*p)); }

// Split over K (blockIdx.z) when there are too few (token, expert) tiles to fill
// the chip: each split writes fp64 partial sums, which the router adds in a fixed
// order before the single rounding to fp32.
template <typename XT>
__global__ __launch_bounds__(256) void gate_logits_f64(const XT* __restrict__ x, const float* __restrict__ wg,
                                                       float* __restrict__ logits, double* __restrict__ partial,
                                                       int T, int E, int H, int kchunk) {
  __shared__ double As[GT][GPAD];
  __shared__ double Bs[GE][GPAD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.y * GT, e0 = blockIdx.x * GE;
  const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

  // loader mapping: thread -> (row = tid / 4, 8 consecutive k at (tid % 4) * 8)
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  const int kbeg = blockIdx.z * kchunk, kend = kbeg + kchunk;
  for (int k0 = kbeg; k0 < kend; k0 += GK) {
    {
      const int t = t0 + lr;
      const bool ok = t < T;
      const XT* src = x + size_t(ok ? t : 0) * H + k0 + lk;
#pragma unroll
      for (int q = 0; q < 8; ++q) As[lr][lk + q] = ok ? load_x64<XT>(src + q) : 0.0;
      const int e = e0 + lr;
      const bool oke = e < E;
      const float* wsrc = wg + size_t(oke ? e : 0) * H + k0 + lk;
#pragma unroll
      for (int q = 0; q < 8; ++q) Bs[lr][lk + q] = oke ? double(wsrc[q]) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < GK / 4; ++s) {
      const int kk = s * 4 + (lane >> 4);
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[wr + i * 16 + (lane & 15)][kk];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[wc + j * 16 + (lane & 15)][kk];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // D[i][j]: lane holds column j = lane % 16, rows 4 * r + lane / 16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wr + i * 16 + r * 4 + (lane >> 4);
        const int e = e0 + wc + j * 16 + (lane & 15);
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
      for (int q = 0; q < nsplit; ++q) z += partial[(size_t(q) * T + t) * E + e];
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
int gate_ksplit(const moe_config_t& c) {
  const int tiles = ((c.num_experts + GE - 1) / GE) * ((c.num_tokens + GT - 1) / GT);
  const int steps = c.hidden / GK;
  int best = 1;
  for (int d = 1; d <= steps && d <= 64; ++d)
    if (steps % d == 0 && tiles * d <= 512) best = d;
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
