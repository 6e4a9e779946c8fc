// Low-precision routed experts on gfx950 scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
//   FP8_B128: weights e4m3fn with an fp32 scale per 128x128 block; activations
//             e4m3fn with an fp32 scale per (row, 128 channels).  The MFMA runs with
//             unit scales over one 128-deep block (two 64-deep steps); the block's
//             partial sums are then multiplied by a_scale[row] * b_scale[col block]
//             and added to the fp32 accumulators.  Block size 128 follows the
//             DeepSeek-V4-Pro overview (lzwjava.github.io, kernel.py: per-block FP8
//             activation quantisation with block 128, FP8 GEMM with per-block A/B
//             scales).
//   MXFP4:    weights e2m1 with an E8M0 scale per 32 along K, activations e4m3fn with
//             an E8M0 scale per 32 (MXFP8): the MFMA applies both scales itself.
//             MXFP4 weights with MXFP8 activations: ruibaoantu.com 2.8T articles,
//             quantisation section; FP4 blocks of 32 with power-of-two scales:
//             V4-Pro overview, kernel.py.
// The SwiGLU output h is re-quantised to the activation format in the epilogue of
// the gate/up GEMM, and is the A operand of the down GEMM.
//
// Operand layout of the 32x32x64 scaled MFMA (measured on gfx950): an fp8
// operand lane (row/column l%32, half h = l/32) holds K = 16h + 0..15 in bytes
// 0..15 and K = 32 + 16h + 0..15 in bytes 16..31; an fp4 operand lane holds
// K = 32h + 0..31 contiguously in 16 bytes, even K in the low nibble.  The E8M0
// scale passed by lane (row i, half h) applies to row i over the natural K
// block [32h, 32h+32).
// fp8 x fp8 (FP8_B128) runs with unit scales, where any K order shared by both
// operands is correct: there lane half h takes k in [64h, 64h+64) of the 128-deep
// step, 64 contiguous weight bytes per lane.  fp8 x fp4 (MXFP4) follows the
// layout above: MFMA sub-step s covers k in [64s, 64s+64), split into the two
// MX blocks 2s and 2s+1.
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

constexpr int QK = 128;   // K per step (fp8 bytes per activation row)

__device__ __forceinline__ int lds_q_off(int r, int c) { return r * QK + ((c ^ (r & 7)) << 4); }

template <int MS, int MODE, int RECIPE>
__global__ __launch_bounds__(256) void ffn_lowp_kernel(GemmArgs g) {
  constexpr int BM = MS * 32;
  constexpr bool MX = RECIPE == MOE_RECIPE_MXFP4;
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * QK];
  __shared__ uint32_t Sa[2][BM];                 // fp32 bits (fp8) or 4 E8M0 bytes (MX)
  __shared__ float amax_lds[4][BM];
  TileInfo ti;
  if (!get_tile(g, BM, ti)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int K = g.K, ns = g.nsplit;
  const uint8_t* A = static_cast<const uint8_t*>(g.A);
  const uint8_t* B = static_cast<const uint8_t*>(g.B);
  constexpr int ELB = MX ? 2 : 1;                // elements per weight byte

  // ---- weight rows (byte pointers) and scale addressing of the two fragments
  const uint8_t* brow[2];
  int ncol[2];                                   // output column of fragment f for this lane
  bool wave_on = true;
  int n0, sub0 = 0;
  if (MODE == EPI_SWIGLU) {
    n0 = blockIdx.x * 128;
    sub0 = ti.e * g.n_experts_split + n0 / ns;
    const int nl = n0 % ns + wave * 32 + l32;
    const uint8_t* base = B + size_t(sub0) * 2 * ns * (K / ELB);
    brow[0] = base + size_t(nl) * (K / ELB);
    brow[1] = base + size_t(ns + nl) * (K / ELB);
    ncol[0] = nl;                                // weight row within the sub-expert
    ncol[1] = ns + nl;
  } else {
    n0 = blockIdx.x * 256;
    wave_on = n0 + wave * 64 < g.N;
    const int n = min(n0 + wave * 64 + l32, g.N - 1);
    const int n1 = min(n + 32, g.N - 1);
    brow[0] = B + size_t(ti.e) * g.n_experts_split * g.N * (ns / ELB) + size_t(n) * (ns / ELB);
    brow[1] = B + size_t(ti.e) * g.n_experts_split * g.N * (ns / ELB) + size_t(n1) * (ns / ELB);
    ncol[0] = n;
    ncol[1] = n1;
  }
  // byte offset of K position k0 within a weight row (down: plus the sub-expert stride)
  auto koff = [&](int k0) -> size_t {
    if (MODE == EPI_SWIGLU) return size_t(k0 / ELB);
    return size_t(k0 / ns) * g.N * (ns / ELB) + (k0 % ns) / ELB;
  };
  // fp8 weight scale of fragment f at K step k0 (uniform across the wave)
  auto bscale_fp8 = [&](int f, int k0) -> float {
    const float* S = static_cast<const float*>(g.B_scale);
    if (MODE == EPI_SWIGLU) {
      const int rb = (f == 0 ? (n0 % ns) : ns + (n0 % ns)) / 128;
      return S[(size_t(sub0) * (2 * ns / 128) + rb) * (K / 128) + k0 / 128];
    }
    const int sub = ti.e * g.n_experts_split + k0 / ns;
    const int cb = (n0 + wave * 64 + f * 32) / 128;
    return S[(size_t(sub) * (g.N / 128) + cb) * (ns / 128) + (k0 % ns) / 128];
  };
  // MX weight scales of fragment f at K step k0: 4 E8M0 bytes (blocks k0/32 .. +3) of this lane's row
  auto bscale_mx = [&](int f, int k0) -> uint32_t {
    const uint8_t* S = static_cast<const uint8_t*>(g.B_scale);
    if (MODE == EPI_SWIGLU)
      return *reinterpret_cast<const uint32_t*>(S + (size_t(sub0) * 2 * ns + ncol[f]) * (K / 32) + k0 / 32);
    const int sub = ti.e * g.n_experts_split + k0 / ns;
    return *reinterpret_cast<const uint32_t*>(S + (size_t(sub) * g.N + ncol[f]) * (ns / 32) + (k0 % ns) / 32);
  };

  f32x16 acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  uint4 areg[MS];
  uint32_t sreg = 0;
  constexpr int BCH = MX ? 2 : 4;                // 16-byte chunks of weight per fragment per step
  uint4 breg[2][BCH];
  auto load_a = [&](int k0) {
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      const int q = tid + 256 * j, r = q >> 3, c = q & 7;
      areg[j] = (r < ti.rows) ? *reinterpret_cast<const uint4*>(A + size_t(ti.row0 + r) * g.lda + k0 + c * 16)
                              : make_uint4(0, 0, 0, 0);
    }
    if (tid < BM) {
      const int r = tid;
      if (MX) {
        const uint8_t* S = static_cast<const uint8_t*>(g.A_scale);
        sreg = (r < ti.rows) ? *reinterpret_cast<const uint32_t*>(S + size_t(ti.row0 + r) * (K / 32) + k0 / 32)
                             : 0x7f7f7f7fu;
      } else {
        const float* S = static_cast<const float*>(g.A_scale);
        sreg = __float_as_uint((r < ti.rows) ? S[size_t(ti.row0 + r) * (K / 128) + k0 / 128] : 0.0f);
      }
    }
  };
  auto store_a = [&](int stg) {
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      const int q = tid + 256 * j, r = q >> 3, c = q & 7;
      *reinterpret_cast<uint4*>(&As[stg][lds_q_off(r, c)]) = areg[j];
    }
    if (tid < BM) Sa[stg][tid] = sreg;
  };
  auto load_b = [&](int k0) {
    if (!wave_on) return;
    if (MX) {                                    // sub-step s: elements 64s + 32h .. +32 = bytes 32s + 16h .. +16
      const size_t o = koff(k0) + half * 16;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int c = 0; c < BCH; ++c) breg[f][c] = *reinterpret_cast<const uint4*>(brow[f] + o + c * 32);
    } else {                                     // 64 contiguous bytes at 64h
      const size_t o = koff(k0) + half * 64;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int c = 0; c < BCH; ++c) breg[f][c] = *reinterpret_cast<const uint4*>(brow[f] + o + c * 16);
    }
  };

  load_a(0);
  load_b(0);
  int stg = 0;
  for (int k0 = 0; k0 < K; k0 += QK) {
    store_a(stg);
    uint4 bcur[2][BCH];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int c = 0; c < BCH; ++c) bcur[f][c] = breg[f][c];
    float sbf[2] = {0.0f, 0.0f};
    uint32_t sbm[2] = {0u, 0u};
    if (wave_on) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (MX) sbm[f] = bscale_mx(f, k0);
        else sbf[f] = bscale_fp8(f, k0);
      }
    }
    if (k0 + QK < K) {
      load_a(k0 + QK);
      load_b(k0 + QK);
    }
    __syncthreads();
    if (wave_on) {
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int ar = i * 32 + l32;
        i32x8 a[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          // fp8 x fp8: bytes 64h + 32s .. +32 of the row; MX: K 64s + 16h .. +16 and 64s + 32 + 16h .. +16
          const int c0 = MX ? 4 * s + half : 4 * half + 2 * s;
          const int c1 = MX ? 4 * s + 2 + half : 4 * half + 2 * s + 1;
          const uint4 lo = *reinterpret_cast<const uint4*>(&As[stg][lds_q_off(ar, c0)]);
          const uint4 hi = *reinterpret_cast<const uint4*>(&As[stg][lds_q_off(ar, c1)]);
          a[s] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
        }
        if (MX) {
          const uint32_t sa4 = Sa[stg][ar];
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const uint4 bw = bcur[f][s];
              const i32x8 b = i32x8{int(bw.x), int(bw.y), int(bw.z), int(bw.w), 0, 0, 0, 0};
              const int sh = 8 * (2 * s + half);  // MX block 2s + h of the 128-deep step
              const int sa = int((sa4 >> sh) & 0xffu), sb = int((sbm[f] >> sh) & 0xffu);
              acc[i][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[s], b, acc[i][f], 0, 4, 0, sa, 0, sb);
            }
        } else {
          float ra[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) ra[r] = __uint_as_float(Sa[stg][i * 32 + acc_row(r, lane)]);
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            f32x16 part;
#pragma unroll
            for (int r = 0; r < 16; ++r) part[r] = 0.0f;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const uint4 b0 = bcur[f][2 * s], b1 = bcur[f][2 * s + 1];
              const i32x8 b = i32x8{int(b0.x), int(b0.y), int(b0.z), int(b0.w), int(b1.x), int(b1.y), int(b1.z), int(b1.w)};
              part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[s], b, part, 0, 0, 0, 127, 0, 127);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][f][r] += part[r] * (ra[r] * sbf[f]);
          }
        }
      }
    }
    stg ^= 1;
  }

  // ---- epilogues
  if (MODE == EPI_SWIGLU) {
    uint8_t* Hq = static_cast<uint8_t*>(g.out);
    const int col = n0 + wave * 32 + l32;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      float hv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) hv[r] = silu_f32(acc[i][0][r]) * acc[i][1][r];
      if (MX) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float amax = max_over_lanes32(fabsf(hv[r]));
          const int row = i * 32 + acc_row(r, lane);
          const int e = mx_exponent_e4m3(amax);
          if (row < ti.rows) {
            Hq[size_t(ti.row0 + row) * g.ldo + col] = uint8_t(f32_to_e4m3(hv[r] * exp2i(-e)));
            if (l32 == 0)
              static_cast<uint8_t*>(g.out_scale)[size_t(ti.row0 + row) * (g.N / 32) + col / 32] = uint8_t(e + 127);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float m = max_over_lanes32(fabsf(hv[r]));
          if (l32 == 0) amax_lds[wave][i * 32 + acc_row(r, lane)] = m;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + acc_row(r, lane);
          const float amax = fmaxf(fmaxf(amax_lds[0][row], amax_lds[1][row]), fmaxf(amax_lds[2][row], amax_lds[3][row]));
          const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
          if (row < ti.rows) {
            Hq[size_t(ti.row0 + row) * g.ldo + col] = uint8_t(f32_to_e4m3(hv[r] / s));
            if (wave == 0 && l32 == 0)
              static_cast<float*>(g.out_scale)[size_t(ti.row0 + row) * (g.N / 128) + n0 / 128] = s;
          }
        }
        __syncthreads();
      }
    }
  } else {
    if (!wave_on) return;
    uint16_t* Y = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int col = n0 + wave * 64 + f * 32 + l32;
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + acc_row(r, lane);
          if (row < ti.rows) Y[size_t(ti.row0 + row) * g.ldo + col] = f32_to_bf16(acc[i][f][r]);
        }
    }
  }
}

template <int MODE, int RECIPE>
static hipError_t launch_lowp_ms(int ms, dim3 grid, const GemmArgs& g, hipStream_t st) {
  switch (ms) {
    case 1: ffn_lowp_kernel<1, MODE, RECIPE><<<grid, 256, 0, st>>>(g); break;
    case 2: ffn_lowp_kernel<2, MODE, RECIPE><<<grid, 256, 0, st>>>(g); break;

    default: ffn_lowp_kernel<4, MODE, RECIPE><<<grid, 256, 0, st>>>(g); break;
  }
  return hipGetLastError();
}

hipError_t launch_lowp_swiglu(int recipe, int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  const dim3 grid(g.N / 128, m_tiles);
  if (recipe == MOE_RECIPE_MXFP4) return launch_lowp_ms<EPI_SWIGLU, MOE_RECIPE_MXFP4>(ms, grid, g, st);
  return launch_lowp_ms<EPI_SWIGLU, MOE_RECIPE_FP8_B128>(ms, grid, g, st);
}

hipError_t launch_lowp_down(int recipe, int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  const dim3 grid((g.N + 255) / 256, m_tiles);
  if (recipe == MOE_RECIPE_MXFP4) return launch_lowp_ms<EPI_STORE, MOE_RECIPE_MXFP4>(ms, grid, g, st);
  return launch_lowp_ms<EPI_STORE, MOE_RECIPE_FP8_B128>(ms, grid, g, st);
}

}  // namespace moe
