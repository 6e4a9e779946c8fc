// post_attention_layernorm in front of the MoE (DeepSeek-V3 walk-through,
// pwwt.cn/news/5781524, section 3.5: the decoder layer normalises the residual
// stream before the MoE and adds the MoE output back; DeepSeek-V4-Pro overview,
// lzwjava.github.io: RMSNorm kept in fp32).
//
// x[t] = act( fp32( (h[t] * r) * w ) ),  r = 1 / sqrt(sum(h[t]^2) / H + eps)
// The squares of bf16/fp32 values are exact in fp64 and the sum, the root and both
// products run in fp64; the value is rounded to fp32 and then to the activation
// format.  Only the summation order differs from the plain definition, which moves
// r by at most a few fp64 ulps.
#include "kernels.h"

namespace moe {

// One 256-thread workgroup per token.  bf16 rows: each thread loads 16-byte chunks
// (8 values) and keeps up to RC of them in registers for the second pass (rows of
// up to 256 * 8 * RC values; longer rows re-read the rest, from L2).
constexpr int RC = 4;

__global__ __launch_bounds__(256) void rmsnorm_bf16(const uint16_t* __restrict__ h, const float* __restrict__ w,
                                                    float eps, int H, uint16_t* __restrict__ x) {
  __shared__ double part[4];
  const uint4* row = reinterpret_cast<const uint4*>(h + size_t(blockIdx.x) * H);
  uint4* out = reinterpret_cast<uint4*>(x + size_t(blockIdx.x) * H);
  const int nc = H / 8;
  uint4 keep[RC];
  double ss = 0.0;
  auto add = [&](uint4 v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double lo = double(__uint_as_float(u[q] << 16)), hi = double(__uint_as_float(u[q] & 0xffff0000u));
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
  };
#pragma unroll
  for (int j = 0; j < RC; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < nc) {
      keep[j] = row[c];
      add(keep[j]);
    }
  }
  for (int c = threadIdx.x + 256 * RC; c < nc; c += 256) add(row[c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double total = (part[0] + part[1]) + (part[2] + part[3]);
  const double r = 1.0 / sqrt(total / double(H) + double(eps));
  auto norm = [&](uint4 v, int c) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    const float4 wa = reinterpret_cast<const float4*>(w)[2 * c], wb = reinterpret_cast<const float4*>(w)[2 * c + 1];
    const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double lo = double(__uint_as_float(u[q] << 16)), hi = double(__uint_as_float(u[q] & 0xffff0000u));
      const float ylo = float((lo * r) * double(wv[2 * q])), yhi = float((hi * r) * double(wv[2 * q + 1]));
      o[q] = uint32_t(f32_to_bf16(ylo)) | (uint32_t(f32_to_bf16(yhi)) << 16);
    }
    out[c] = uint4{o[0], o[1], o[2], o[3]};
  };
#pragma unroll
  for (int j = 0; j < RC; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < nc) norm(keep[j], c);
  }
  for (int c = threadIdx.x + 256 * RC; c < nc; c += 256) norm(row[c], c);
}

// fp32 rows (the fp32 recipe's small shapes): plain per-element loops.
__global__ __launch_bounds__(256) void rmsnorm_f32(const float* __restrict__ h, const float* __restrict__ w, float eps,
                                                   int H, float* __restrict__ x) {
  __shared__ double part[4];
  const size_t base = size_t(blockIdx.x) * H;
  double ss = 0.0;
  for (int i = threadIdx.x; i < H; i += 256) {
    const double v = double(h[base + i]);
    ss = fma(v, v, ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double total = (part[0] + part[1]) + (part[2] + part[3]);
  const double r = 1.0 / sqrt(total / double(H) + double(eps));
  for (int i = threadIdx.x; i < H; i += 256) x[base + i] = float((double(h[base + i]) * r) * double(w[i]));
}

hipError_t launch_rmsnorm(const moe_config_t& c, const void* h, const float* w, float eps, void* x, hipStream_t st) {
  ProfScope p(MOE_K_RMSNORM, st);
  if (c.recipe == MOE_RECIPE_F32)
    rmsnorm_f32<<<c.num_tokens, 256, 0, st>>>(static_cast<const float*>(h), w, eps, c.hidden, static_cast<float*>(x));
  else                                                 // hidden % 128 == 0: whole 16-byte chunks
    rmsnorm_bf16<<<c.num_tokens, 256, 0, st>>>(static_cast<const uint16_t*>(h), w, eps, c.hidden,
                                               static_cast<uint16_t*>(x));
  return hipGetLastError();
}

}  // namespace moe
