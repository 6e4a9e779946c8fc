// moe_infer's "count tokens per expert, argsort by expert id into contiguous
// blocks" (DeepSeek-V3 walk-through, pwwt.cn/news/5781524, section 3.4) as a
// deterministic counting sort, plus the row gather into that order.
//
// The sort is stable over the flat pair index f = t*k + j:
//   perm_hist    per chunk of PERM_CHUNK pairs, an LDS histogram over experts;
//   perm_scan    per expert, prefix over chunks; exclusive scan over experts;
//   perm_scatter one wavefront per chunk walks its pairs in order, 64 at a time,
//                ranking equal experts inside the wave with ballots (no atomics),
//                so every row position is fixed by (expert, f) alone.
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void perm_hist(const int32_t* __restrict__ idx, int pairs, int E,
                                                 int32_t* __restrict__ hist) {
  __shared__ int32_t h[1024];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * PERM_CHUNK;
  for (int q = threadIdx.x; q < PERM_CHUNK; q += 256) {
    const int f = base + q;
    if (f < pairs) atomicAdd(&h[idx[f]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[size_t(blockIdx.x) * E + e] = h[e];
}

// One block of 1024 threads; E <= 1024.  hist[b][e] becomes the first row of
// chunk b's pairs of expert e; offsets[E+1] the expert block starts.
__global__ __launch_bounds__(1024) void perm_scan(int32_t* __restrict__ hist, int nb, int E,
                                                  int32_t* __restrict__ offsets) {
  __shared__ int32_t cnt[1024];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nb; ++b) {
      const int v = hist[size_t(b) * E + e];
      hist[size_t(b) * E + e] = run;
      run += v;
    }
  }
  cnt[e] = (e < E) ? run : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over 1024 entries
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = (e >= off) ? cnt[e - off] : 0;
    __syncthreads();
    cnt[e] += v;
    __syncthreads();
  }
  const int excl = cnt[e] - ((e < E) ? run : 0);
  if (e < E) {
    offsets[e] = excl;
    for (int b = 0; b < nb; ++b) hist[size_t(b) * E + e] += excl;
  }
  if (e == E - 1) offsets[E] = cnt[e];
}

__global__ __launch_bounds__(64) void perm_scatter(const int32_t* __restrict__ idx, int pairs, int E,
                                                   const int32_t* __restrict__ hist, int32_t* __restrict__ sorted_pair,
                                                   int32_t* __restrict__ pair_pos) {
  __shared__ int32_t run[1024];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) run[e] = hist[size_t(blockIdx.x) * E + e];
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int base = blockIdx.x * PERM_CHUNK;
  for (int step = 0; step < PERM_CHUNK; step += 64) {
    const int f = base + step + lane;
    const bool ok = f < pairs;
    const int e = ok ? idx[f] : 0;
    uint64_t match = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    const int rank = __popcll(match & lt);
    const int pos = run[e] + rank;                       // every lane reads before any update
    __syncthreads();
    if (ok) {
      sorted_pair[pos] = f;
      pair_pos[f] = pos;
      if (64 - __clzll(match) - 1 == lane) run[e] = pos + 1;   // highest lane of its group
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Gather x rows into the sorted order, in the routed-activation format.
// One wavefront per destination row; each lane owns 8 consecutive channels.
// ---------------------------------------------------------------------------
template <int RECIPE>
__global__ __launch_bounds__(256) void perm_gather(const void* __restrict__ xv, const int32_t* __restrict__ sorted_pair,
                                                   int pairs, int k, int H, void* __restrict__ outv,
                                                   void* __restrict__ scalev) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + wave;
  if (p >= pairs) return;
  const int t = sorted_pair ? sorted_pair[p] / k : p;   // (no pair order: quantise token rows in place order)
  if (RECIPE == MOE_RECIPE_F32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + size_t(t) * H);
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(outv) + size_t(p) * H);
    for (int c = lane; c < H / 4; c += 64) dst[c] = src[c];
    return;
  }
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + size_t(t) * H);
  if (RECIPE == MOE_RECIPE_BF16) {
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(outv) + size_t(p) * H);
    for (int c = lane; c < H / 8; c += 64) dst[c] = src[c];
    return;
  }
  if (RECIPE == MOE_RECIPE_NVFP4) {                   // fp16 values of the NVFP4 rows: 16 channels = 2 lanes
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(outv) + size_t(p) * H);
    for (int c0 = 0; c0 < H / 8; c0 += 64) {
      const int c = c0 + lane;
      const bool ok = c < H / 8;                       // H % 128 == 0: lane pairs are all-or-none
      const uint4 raw = ok ? src[c] : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      float v[8], amax = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      const float s = nvfp4_scale(amax);
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x2 pr = {_Float16(nvfp4_value(v[2 * q], s)), _Float16(nvfp4_value(v[2 * q + 1], s))};
        o[q] = __builtin_bit_cast(uint32_t, pr);
      }
      if (ok) dst[c] = uint4{o[0], o[1], o[2], o[3]};
    }
    return;
  }
  // fp8 codes: lane handles 8 channels -> 8 bytes
  uint2* dst = reinterpret_cast<uint2*>(static_cast<uint8_t*>(outv) + size_t(p) * H);
  for (int c0 = 0; c0 < H / 8; c0 += 64) {              // 512 channels per pass
    const int c = c0 + lane;
    const bool ok = c < H / 8;                           // H % 128 == 0: groups of 16 lanes are all-or-none
    uint4 raw = ok ? src[c] : make_uint4(0, 0, 0, 0);
    float v[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
    uint32_t code[8];
    if (RECIPE == MOE_RECIPE_FP8_B128) {                 // 128 channels = 16 lanes
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) code[q] = f32_to_e4m3(v[q] / s);
      if (ok && (lane & 15) == 0) static_cast<float*>(scalev)[size_t(p) * (H / 128) + c / 16] = s;
    } else {                                             // MXFP8: 32 channels = 4 lanes
#pragma unroll
      for (int off = 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      const int e = mx_exponent_e4m3(amax);
      const float inv = exp2i(-e);
#pragma unroll
      for (int q = 0; q < 8; ++q) code[q] = f32_to_e4m3(v[q] * inv);
      if (ok && (lane & 3) == 0) static_cast<uint8_t*>(scalev)[size_t(p) * (H / 32) + c / 4] = uint8_t(e + 127);
    }
    if (ok) {
      uint2 o;
      o.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
      o.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
      dst[c] = o;
    }
  }
}

hipError_t launch_permute(const moe_config_t& c, const int32_t* topk_idx, const void* x, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, void* x_perm, void* x_perm_scale,
                          int32_t* hist_ws, hipStream_t st) {
  const int pairs = c.num_tokens * c.top_k, E = c.num_experts, nb = perm_blocks(pairs);
  {
    ProfScope p(MOE_K_PERM_HIST, st);
    perm_hist<<<nb, 256, 0, st>>>(topk_idx, pairs, E, hist_ws);
  }
  {
    ProfScope p(MOE_K_PERM_SCAN, st);
    perm_scan<<<1, 1024, 0, st>>>(hist_ws, nb, E, offsets);
  }
  {
    ProfScope p(MOE_K_PERM_SCATTER, st);
    perm_scatter<<<nb, 64, 0, st>>>(topk_idx, pairs, E, hist_ws, sorted_pair, pair_pos);
  }
  if (x_perm) {
    ProfScope p(MOE_K_GATHER, st);
    const int g = (pairs + 3) / 4;
    switch (c.recipe) {
      case MOE_RECIPE_F32:
        perm_gather<MOE_RECIPE_F32><<<g, 256, 0, st>>>(x, sorted_pair, pairs, c.top_k, c.hidden, x_perm, nullptr);
        break;
      case MOE_RECIPE_BF16:
        perm_gather<MOE_RECIPE_BF16><<<g, 256, 0, st>>>(x, sorted_pair, pairs, c.top_k, c.hidden, x_perm, nullptr);
        break;
      case MOE_RECIPE_FP8_B128:
        perm_gather<MOE_RECIPE_FP8_B128><<<g, 256, 0, st>>>(x, sorted_pair, pairs, c.top_k, c.hidden, x_perm,
                                                             x_perm_scale);
        break;
      case MOE_RECIPE_NVFP4:
        perm_gather<MOE_RECIPE_NVFP4><<<g, 256, 0, st>>>(x, sorted_pair, pairs, c.top_k, c.hidden, x_perm, nullptr);
        break;
      default:
        perm_gather<MOE_RECIPE_MXFP4><<<g, 256, 0, st>>>(x, sorted_pair, pairs, c.top_k, c.hidden, x_perm,
                                                          x_perm_scale);
    }
  }
  return hipGetLastError();
}

// Activation quantisation of the token rows in token order (the fused-gather path:
// the grouped GEMMs then read row token(p) of this copy for pair row p).
hipError_t launch_quantize_tokens(const moe_config_t& c, const void* x, void* xq, void* xq_scale, hipStream_t st) {
  ProfScope p(MOE_K_GATHER, st);
  const int g = (c.num_tokens + 3) / 4;
  if (c.recipe == MOE_RECIPE_FP8_B128)
    perm_gather<MOE_RECIPE_FP8_B128><<<g, 256, 0, st>>>(x, nullptr, c.num_tokens, 1, c.hidden, xq, xq_scale);
  else if (c.recipe == MOE_RECIPE_MXFP4)
    perm_gather<MOE_RECIPE_MXFP4><<<g, 256, 0, st>>>(x, nullptr, c.num_tokens, 1, c.hidden, xq, xq_scale);
  else if (c.recipe == MOE_RECIPE_NVFP4)
    perm_gather<MOE_RECIPE_NVFP4><<<g, 256, 0, st>>>(x, nullptr, c.num_tokens, 1, c.hidden, xq, nullptr);
  return hipGetLastError();
}

}  // namespace moe
