// Tile lists for the grouped GEMMs, the fp32 expert MLP (VALU), and the
// weighted put-back sum of the routed rows (plus the shared-expert rows).
// moe_infer per-expert MLP and put-back: DeepSeek-V3 walk-through
// (pwwt.cn/news/5781524), section 3.4.
#include <algorithm>

#include "gemm_common.h"
#include "kernels.h"

namespace moe {

// Two tile lists, {count, e_0, m0_0, e_1, m0_1, ...} each: experts with at least
// `thresh` rows are cut into bm_large-row tiles (list L), the others into
// bm_small-row tiles (list S).
__global__ __launch_bounds__(1024) void build_tiles2(const int32_t* __restrict__ offsets, int E, int thresh,
                                                     int bm_large, int bm_small, int32_t* __restrict__ tiles_l,
                                                     int32_t* __restrict__ tiles_s) {
  __shared__ int32_t cl[1024], cs[1024];
  const int e = threadIdx.x;
  const int m = (e < E) ? offsets[e + 1] - offsets[e] : 0;
  const bool large = m >= thresh;
  const int nl = large ? (m + bm_large - 1) / bm_large : 0;
  const int nsm = large ? 0 : (m + bm_small - 1) / bm_small;
  cl[e] = nl;
  cs[e] = nsm;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int vl = (e >= off) ? cl[e - off] : 0;
    const int vs = (e >= off) ? cs[e - off] : 0;
    __syncthreads();
    cl[e] += vl;
    cs[e] += vs;
    __syncthreads();
  }
  const int fl = cl[e] - nl, fs = cs[e] - nsm;
  for (int q = 0; q < nl; ++q) {
    tiles_l[1 + 2 * (fl + q)] = e;
    tiles_l[2 + 2 * (fl + q)] = q * bm_large;
  }
  for (int q = 0; q < nsm; ++q) {
    tiles_s[1 + 2 * (fs + q)] = e;
    tiles_s[2 + 2 * (fs + q)] = q * bm_small;
  }
  if (e == 1023) {
    tiles_l[0] = cl[1023];
    tiles_s[0] = cs[1023];
  }
}

// ---------------------------------------------------------------------------
// fp32 expert MLP on the vector ALU: one thread per output element, 16 x 16 per block.
// ---------------------------------------------------------------------------
constexpr int F32_BM = 16;

template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(GemmArgs g) {
  TileInfo ti;
  if (!get_tile(g, F32_BM, ti)) return;
  const int r = threadIdx.x >> 4;
  const int col = blockIdx.x * 16 + (threadIdx.x & 15);
  if (r >= ti.rows || col >= g.N) return;
  const float* A = static_cast<const float*>(g.A) + size_t(a_row(g, ti.row0 + r)) * g.lda;
  const float* B = static_cast<const float*>(g.B);
  const int K = g.K, ns = g.nsplit;
  if (MODE == EPI_SWIGLU) {
    const int sub = ti.e * g.n_experts_split + col / ns, nl = col % ns;
    const float* wg = B + size_t(sub) * 2 * ns * K + size_t(nl) * K;
    const float* wu = wg + size_t(ns) * K;
    float a0 = 0.0f, a1 = 0.0f;
    for (int k = 0; k < K; ++k) {
      a0 = fmaf(A[k], wg[k], a0);
      a1 = fmaf(A[k], wu[k], a1);
    }
    static_cast<float*>(g.out)[size_t(ti.row0 + r) * g.ldo + col] = swiglu_f32(a0, a1, g.swiglu_limit);
    return;
  }
  float acc = 0.0f;
  for (int k0 = 0; k0 < K; k0 += ns) {                 // down_proj, one sub-expert at a time
    const int sub = ti.e * g.n_experts_split + k0 / ns;
    const float* w = B + size_t(sub) * g.N * ns + size_t(col) * ns;
    for (int k = 0; k < ns; ++k) acc = fmaf(A[k0 + k], w[k], acc);
  }
  if (MODE == EPI_STORE) {
    static_cast<float*>(g.out)[size_t(ti.row0 + r) * g.ldo + col] = acc;
  } else {
    const int t = ti.row0 + r, k = g.topk;
    const float* Yp = static_cast<const float*>(g.y_perm);
    if (g.resid) acc += static_cast<const float*>(g.resid)[size_t(t) * g.ldo + col];
    for (int j = 0; j < k; ++j)
      acc += g.topk_w[size_t(t) * k + j] * Yp[size_t(g.pair_pos[size_t(t) * k + j]) * g.ldo + col];
    static_cast<float*>(g.out)[size_t(t) * g.ldo + col] = acc;
  }
}

hipError_t launch_f32(int mode, int m_tiles, const GemmArgs& g, hipStream_t st) {
  const dim3 grid((g.N + 15) / 16, m_tiles);
  if (mode == EPI_SWIGLU) ffn_f32_kernel<EPI_SWIGLU><<<grid, 256, 0, st>>>(g);
  else if (mode == EPI_STORE) ffn_f32_kernel<EPI_STORE><<<grid, 256, 0, st>>>(g);
  else ffn_f32_kernel<EPI_COMBINE><<<grid, 256, 0, st>>>(g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Put back + weighted sum (+ shared experts):
//   out[t] = sum_j w[t][j] * y_perm[pair_pos[t*k+j]] (+ sh[t]), fp32 accumulation.
// One workgroup per token; each thread owns 8 consecutive channels (16-byte loads).
// ---------------------------------------------------------------------------
// sh: nsh fp32 slabs [T][H], sh_stride elements apart, summed in order (K-split
// partial products of the shared expert's down projection; nsh = 1: its rows).
// resid (nullable): bf16 residual rows [T][H], added first.  out may alias resid:
// each thread reads its 8 channels of resid before writing them.
__global__ __launch_bounds__(256) void combine_bf16(const uint16_t* __restrict__ yp, const int32_t* __restrict__ pair_pos,
                                                    const float* __restrict__ w, const float* __restrict__ sh, int nsh,
                                                    size_t sh_stride, int k, int H, const uint16_t* resid,
                                                    uint16_t* out) {
  __shared__ int32_t pos[16];
  __shared__ float wt[16];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    pos[threadIdx.x] = pair_pos[size_t(t) * k + threadIdx.x];
    wt[threadIdx.x] = w[size_t(t) * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    if (resid) {
      const uint4 v = reinterpret_cast<const uint4*>(resid + size_t(t) * H)[c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = __uint_as_float(u[q] << 16);
        acc[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
      }
    }
    for (int z = 0; z < nsh; ++z) {
      const float4* src = reinterpret_cast<const float4*>(sh + z * sh_stride + size_t(t) * H);
      const float4 a = src[2 * c], b = src[2 * c + 1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w; acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    for (int j = 0; j < k; ++j) {
      const uint4 v = reinterpret_cast<const uint4*>(yp + size_t(pos[j]) * H)[c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      const float wj = wt[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += wj * __uint_as_float(u[q] << 16);
        acc[2 * q + 1] += wj * __uint_as_float(u[q] & 0xffff0000u);
      }
    }
    uint4 o;
    o.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
    o.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
    o.z = uint32_t(f32_to_bf16(acc[4])) | (uint32_t(f32_to_bf16(acc[5])) << 16);
    o.w = uint32_t(f32_to_bf16(acc[6])) | (uint32_t(f32_to_bf16(acc[7])) << 16);
    reinterpret_cast<uint4*>(out + size_t(t) * H)[c] = o;
  }
}

__global__ __launch_bounds__(256) void combine_f32(const float* __restrict__ yp, const int32_t* __restrict__ pair_pos,
                                                   const float* __restrict__ w, int k, int H, const float* resid,
                                                   float* out) {
  const int t = blockIdx.x;
  for (int n = threadIdx.x; n < H; n += 256) {
    float acc = resid ? resid[size_t(t) * H + n] : 0.0f;
    for (int j = 0; j < k; ++j) acc += w[size_t(t) * k + j] * yp[size_t(pair_pos[size_t(t) * k + j]) * H + n];
    out[size_t(t) * H + n] = acc;
  }
}

// sh: nsh fp32 slabs of shared-expert rows [T][H] (bf16-output recipes only; nsh = 0: none).
hipError_t launch_combine_rows(const moe_config_t& c, const void* y_perm, const int32_t* pair_pos,
                               const float* topk_w, const float* sh, int nsh, const void* resid, void* out,
                               hipStream_t st) {
  if (c.recipe == MOE_RECIPE_F32)
    combine_f32<<<c.num_tokens, 256, 0, st>>>(static_cast<const float*>(y_perm), pair_pos, topk_w, c.top_k,
                                              c.hidden, static_cast<const float*>(resid), static_cast<float*>(out));
  else
    combine_bf16<<<c.num_tokens, 256, 0, st>>>(static_cast<const uint16_t*>(y_perm), pair_pos, topk_w, sh, nsh,
                                               size_t(c.num_tokens) * c.hidden, c.top_k, c.hidden,
                                               static_cast<const uint16_t*>(resid), static_cast<uint16_t*>(out));
  return hipGetLastError();
}

// SwiGLU of K-split gate/up partial products: part holds nz fp32 slabs [T][nes*2*Is]
// (sub-expert s: gate columns s*2Is .. +Is, up columns s*2Is+Is .. +Is), summed in
// order; h[t][s*Is + c] = bf16(SiLU(gate) * up).
__global__ __launch_bounds__(256) void swiglu_slabs(const float* __restrict__ part, int nz, int T, int nes, int Is,
                                                    float limit, uint16_t* __restrict__ h) {
  const int SI = nes * Is;
  const size_t stride = size_t(T) * 2 * SI;
  const size_t n4 = size_t(T) * SI / 4;
  for (size_t q = size_t(blockIdx.x) * 256 + threadIdx.x; q < n4; q += size_t(gridDim.x) * 256) {
    const size_t i = q * 4;
    const int t = int(i / SI), col = int(i % SI), s = col / Is, c = col % Is;
    const size_t gi = size_t(t) * 2 * SI + size_t(s) * 2 * Is + c;
    float4 gs = make_float4(0.f, 0.f, 0.f, 0.f), us = gs;
    for (int z = 0; z < nz; ++z) {
      const float4 gv = *reinterpret_cast<const float4*>(part + z * stride + gi);
      const float4 uv = *reinterpret_cast<const float4*>(part + z * stride + gi + Is);
      gs.x += gv.x; gs.y += gv.y; gs.z += gv.z; gs.w += gv.w;
      us.x += uv.x; us.y += uv.y; us.z += uv.z; us.w += uv.w;
    }
    uint2 o;
    o.x = uint32_t(f32_to_bf16(swiglu_f32(gs.x, us.x, limit))) | (uint32_t(f32_to_bf16(swiglu_f32(gs.y, us.y, limit))) << 16);
    o.y = uint32_t(f32_to_bf16(swiglu_f32(gs.z, us.z, limit))) | (uint32_t(f32_to_bf16(swiglu_f32(gs.w, us.w, limit))) << 16);
    *reinterpret_cast<uint2*>(h + i) = o;
  }
}

hipError_t launch_swiglu_slabs(const float* part, int nz, int T, int nes, int Is, float limit, uint16_t* h,
                               hipStream_t st) {
  const size_t n4 = size_t(T) * nes * Is / 4;
  const int blocks = int(std::min<size_t>((n4 + 255) / 256, 2048));
  swiglu_slabs<<<blocks, 256, 0, st>>>(part, nz, T, nes, Is, limit, h);
  return hipGetLastError();
}

hipError_t launch_build_tiles2(const int32_t* offsets, int E, int thresh, int bm_large, int bm_small,
                               int32_t* tiles_l, int32_t* tiles_s, hipStream_t st) {
  build_tiles2<<<1, 1024, 0, st>>>(offsets, E, thresh, bm_large, bm_small, tiles_l, tiles_s);
  return hipGetLastError();
}

}  // namespace moe
