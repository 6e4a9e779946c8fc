// Per-expert SwiGLU MLP of moe_infer (DeepSeek-V3 walk-through, pwwt.cn/news/5781524,
// section 3.4: each expert runs gate/up/down + SiLU over its contiguous block),
// as a grouped bf16 MFMA GEMM on gfx950, and the shared expert(s) of
// DeepseekV3MoE.forward (their down projection stores fp32 rows for the put-back sum).
//
// Tile: BM = 32*MS rows x (SwiGLU: 128 h columns | down: 256 output columns),
// four wavefronts.  The rows (activations) are staged through LDS, shared by the
// four waves; each wave streams its own weight rows straight from HBM into
// registers in the MFMA B-operand layout, so every weight byte of a tile is read
// exactly once.  K advances 64 per step with a two-stage LDS ring.
//
// MFMA v_mfma_f32_32x32x16_bf16: lane l of the A operand holds row l%32, and of
// the B operand column l%32; both hold 8 K-values chosen by l/32.  Any
// permutation of K that is the same for A and B gives the same product, so lane
// half h of step s takes k = k0 + 32h + 8s .. +8: each lane then reads 64
// contiguous weight bytes per step.
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

constexpr int BK = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// LDS A tile: BM rows x 64 bf16 = 8 chunks of 16 bytes per row; chunk c of row r
// lives at chunk slot c ^ (r & 7) so that the 8 rows a read phase touches hit
// distinct banks.
__device__ __forceinline__ int lds_a_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

template <int MS, int MODE>
__global__ __launch_bounds__(256) void ffn_bf16_kernel(GemmArgs g) {
  constexpr int BM = MS * 32;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  TileInfo ti;
  if (!get_tile(g, BM, ti)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int K = g.K, ns = g.nsplit;
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* B = static_cast<const uint16_t*>(g.B);

  // ---- weight rows of this wave's two fragments
  const uint16_t* brow[2];
  bool wave_on = true;
  int n0;
  if (MODE == EPI_SWIGLU) {
    n0 = blockIdx.x * 128;
    const int sub = ti.e * g.n_experts_split + n0 / ns;
    const int nl = n0 % ns + wave * 32 + l32;
    const uint16_t* base = B + size_t(sub) * 2 * ns * K;
    brow[0] = base + size_t(nl) * K;             // gate_proj row
    brow[1] = base + size_t(ns + nl) * K;        // up_proj row
  } else {
    n0 = blockIdx.x * 256;
    wave_on = n0 + wave * 64 < g.N;
    const int n = min(n0 + wave * 64 + l32, g.N - 1);
    brow[0] = B + size_t(ti.e) * g.n_experts_split * g.N * ns + size_t(n) * ns;
    brow[1] = brow[0] + size_t(min(32, g.N - 1 - n)) * ns;   // column n + 32 (clamped when inactive)
  }
  auto koff = [&](int k0) -> size_t {
    if (MODE == EPI_SWIGLU) return size_t(k0);
    return size_t(k0 / ns) * g.N * ns + (k0 % ns);            // down_proj of the sub-expert owning k0
  };

  f32x16 acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  uint4 areg[MS];
  uint4 breg[2][4];
  auto load_a = [&](int k0) {
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      const int q = tid + 256 * j, r = q >> 3, c = q & 7;
      areg[j] = (r < ti.rows) ? *reinterpret_cast<const uint4*>(A + size_t(ti.row0 + r) * g.lda + k0 + c * 8)
                              : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int stg) {
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      const int q = tid + 256 * j, r = q >> 3, c = q & 7;
      *reinterpret_cast<uint4*>(&As[stg][lds_a_off(r, c)]) = areg[j];
    }
  };
  auto load_b = [&](int k0) {
    if (!wave_on) return;
    const size_t o = koff(k0) + half * 32;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int s = 0; s < 4; ++s) breg[f][s] = *reinterpret_cast<const uint4*>(brow[f] + o + s * 8);
  };

  load_a(0);
  load_b(0);
  int stg = 0;
  for (int k0 = 0; k0 < K; k0 += BK) {
    store_a(stg);
    uint4 bcur[2][4];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int s = 0; s < 4; ++s) bcur[f][s] = breg[f][s];
    if (k0 + BK < K) {
      load_a(k0 + BK);
      load_b(k0 + BK);
    }
    __syncthreads();
    if (wave_on) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 b0 = as_bf16x8(bcur[0][s]), b1 = as_bf16x8(bcur[1][s]);
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&As[stg][lds_a_off(i * 32 + l32, half * 4 + s)]));
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[i][1], 0, 0, 0);
        }
      }
    }
    stg ^= 1;
  }
  if (!wave_on) return;

  // ---- epilogues
  if (MODE == EPI_SWIGLU) {
    uint16_t* H = static_cast<uint16_t*>(g.out);
    const int col = n0 + wave * 32 + l32;
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + acc_row(r, lane);
        if (row < ti.rows) {
          const float gt = acc[i][0][r], up = acc[i][1][r];
          H[size_t(ti.row0 + row) * g.ldo + col] = f32_to_bf16(silu_f32(gt) * up);
        }
      }
  } else {  // EPI_STORE: bf16 y rows, or fp32 rows (out_f32)
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int col = n0 + wave * 64 + f * 32 + l32;
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + acc_row(r, lane);
          if (row >= ti.rows) continue;
          const size_t o = size_t(ti.row0 + row) * g.ldo + col;
          if (g.out_f32) static_cast<float*>(g.out)[o] = acc[i][f][r];
          else static_cast<uint16_t*>(g.out)[o] = f32_to_bf16(acc[i][f][r]);
        }
    }
  }
}

// Rows per tile for a grouped launch: about the mean rows per expert, so that few
// rows of a tile are padding.
template <int MODE>
static hipError_t launch_ms(int ms, dim3 grid, const GemmArgs& g, hipStream_t st) {
  switch (ms) {
    case 1: ffn_bf16_kernel<1, MODE><<<grid, 256, 0, st>>>(g); break;
    case 2: ffn_bf16_kernel<2, MODE><<<grid, 256, 0, st>>>(g); break;

    default: ffn_bf16_kernel<4, MODE><<<grid, 256, 0, st>>>(g); break;
  }
  return hipGetLastError();
}

hipError_t launch_bf16_swiglu(int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  return launch_ms<EPI_SWIGLU>(ms, dim3(g.N / 128, m_tiles), g, st);
}
hipError_t launch_bf16_down(int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  return launch_ms<EPI_STORE>(ms, dim3((g.N + 255) / 256, m_tiles), g, st);
}

}  // namespace moe
