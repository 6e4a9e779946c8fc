// Grouped expert GEMMs for experts with few rows (decode, fine-grained and the long
// tail of a skewed load): moe_infer's per-expert gate/up/down + SiLU
// (DeepSeek-V3 walk-through, pwwt.cn/news/5781524, section 3.4) where the time
// goes into streaming each expert's weights once from HBM.
//
// Tile: 32*MS rows x 256 weight rows (SwiGLU: 128 gate_proj + the matching 128
// up_proj rows; down: 256 output columns); four wavefronts, wave w owns every row
// and weight rows [32w, 32w+32) of each half.  Weights go straight from HBM into
// MFMA B-operand registers through a ring of NST register stages (NST-1 stages in
// flight per wave), each lane reading 64 contiguous bytes per fragment and stage;
// the few activation rows go through a matching LDS ring filled by async
// global->LDS copies.  Small register footprint -> several waves per SIMD, so
// plenty of weight bytes are in flight per CU.
//
// Recipes:
//   bf16      v_mfma_f32_32x32x16_bf16, K = 64 per stage.  Lane half h of step s
//             takes k = 32h + 8s .. +8 (A and B alike).
//   fp8_b128  v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales, K = 128 per stage
//             (one 128x128 scale block); lane half h of sub-step s takes bytes
//             64h + 32s .. +32; acc += part * a_scale[row] * b_scale[block].
//   mxfp4     the same MFMA with fp8 activations x fp4 weights and per-32 E8M0
//             scales on both operands, K = 128 per stage.  Operand layout measured
//             on gfx950: an fp8 operand lane (half h) holds K = 16h + 0..15 and
//             32 + 16h + 0..15, an fp4 operand lane holds K = 32h + 0..31 (even K in
//             the low nibble), and the scale of lane (row, h) applies to K block h.
//   nvfp4     v_mfma_f32_32x32x16_f16 on exactly dequantised operands: activations
//             arrive as the fp16 values of their NVFP4 quantisation; e2m1 weights
//             are turned into fp16 in registers (byte lookup of the fp16 high byte,
//             times the group's e4m3 scale: every such product is exact in fp16).
// The SwiGLU output h is written as bf16, or re-quantised to the activation format
// (NVFP4: stored as fp16 values).
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int RS_ROWB = 128;     // activation bytes of K per LDS row and stage
constexpr int RS_NB = 256;       // weight rows per tile

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int rs_slot(int r, int c) { return c ^ ((r ^ (r >> 1)) & 7); }
__device__ __forceinline__ int rs_swz(int r, int c) { return r * RS_ROWB + (rs_slot(r, c) << 4); }

template <int N>
__device__ __forceinline__ void rs_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

__device__ __forceinline__ void rs_copy16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// Eight e2m1 codes (one dword, low nibble = lower k) times an fp16 scale pair ->
// eight fp16 values in k order.  The magnitudes index a byte table of the fp16
// high bytes (the low byte of every e2m1 value in fp16 is zero); the sign bit of
// each nibble becomes the fp16 sign.
__device__ __forceinline__ f16x8 e2m1x8_to_f16(uint32_t w, f16x2 scale) {
  constexpr uint32_t T_LO = 0x3E3C3800u, T_HI = 0x46444240u;   // 0, .5, 1, 1.5 | 2, 3, 4, 6
  const uint32_t he = __builtin_amdgcn_perm(T_HI, T_LO, w & 0x07070707u) | ((w << 4) & 0x80808080u);   // even k
  const uint32_t ho = __builtin_amdgcn_perm(T_HI, T_LO, (w >> 4) & 0x07070707u) | (w & 0x80808080u);   // odd k
  f16x8 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // bytes: 0, even k = 2q high byte, 0, odd k = 2q+1 high byte
    const uint32_t d = __builtin_amdgcn_perm(ho, he, 0x040C000Cu + 0x01000100u * q);
    const f16x2 v = __builtin_bit_cast(f16x2, d) * scale;
    out[2 * q] = v[0];
    out[2 * q + 1] = v[1];
  }
  return out;
}

__device__ __forceinline__ i32x8 rs_cat(uint4 lo, uint4 hi) {
  return i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

}  // namespace

// WPE: minimum waves per SIMD the register allocation must leave room for.
template <int MS, int MODE, int RECIPE, int NST, int WPE = 1>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) void ffn_rs_kernel(GemmArgs g) {
  constexpr int BM = MS * 32;
  constexpr bool BF16 = RECIPE == MOE_RECIPE_BF16;
  constexpr bool MX = RECIPE == MOE_RECIPE_MXFP4;
  constexpr bool FP8 = RECIPE == MOE_RECIPE_FP8_B128;
  constexpr bool NV = RECIPE == MOE_RECIPE_NVFP4;
  constexpr bool FP4 = MX || NV;                   // packed e2m1 weights with per-row scale bytes
  constexpr bool ASC = FP8 || MX;                  // activations as codes plus row scales
  constexpr int EA = (BF16 || NV) ? 2 : 1;         // activation bytes per element (NVFP4: fp16 values)
  constexpr int KS = RS_ROWB / EA;                 // K per stage
  constexpr int WB = FP4 ? 2 : 1;                  // weight elements per byte (fp4: 2)
  constexpr int EBW = BF16 ? 2 : 1;                // weight bytes per element (bf16 2, fp8 1; fp4 via WB)
  constexpr int BCH = MX ? 2 : (NV ? 1 : 4);       // 16-byte weight chunks per fragment and stage
  constexpr int SG = MX ? 32 : 16;                 // fp4 scale group along K
  constexpr int A_INSTR = MS;                      // async copies per wave per stage: BM*8 chunks / 256 lanes
  __shared__ __attribute__((aligned(1024))) uint8_t As[NST][BM * RS_ROWB];
  __shared__ uint32_t Sa[NST][BM];                 // fp8: fp32 row scale bits; MX: 4 E8M0 bytes
  __shared__ float amax_lds[4][BM];

  // (row tile, column block) pairs in XCD-major order: one expert's row tiles and
  // column blocks run on one XCD, which then reads its weights and activations once
  const int ncols = int(gridDim.x);
  const int V = ncols * row_tiles(g, BM);
  const int b = int(blockIdx.y) * ncols + int(blockIdx.x);
  if (b >= V) return;
  const int tnum = xcd_tile(b, V), mt = tnum / ncols, nt = tnum - mt * ncols;
  TileInfo ti;
  if (!tile_info(g, BM, mt, ti)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int K = g.K, ns = g.nsplit;
  const uint8_t* A = static_cast<const uint8_t*>(g.A);
  const uint8_t* B = static_cast<const uint8_t*>(g.B);
  const int act_ms = (ti.rows + 31) >> 5;

  // ---- this lane's weight rows (byte pointers) of fragments 0 and 1
  const uint8_t* brow[2];
  int ncol[2];                                     // weight row index within its matrix (for MX scales)
  bool wave_on = true;
  int n0, sub0 = 0;
  if (MODE == EPI_SWIGLU) {
    n0 = nt * 128;
    sub0 = ti.e * g.n_experts_split + n0 / ns;
    const int nl = n0 % ns + wave * 32 + l32;
    const size_t rowbytes = FP4 ? size_t(K) / 2 : size_t(K) * EBW;
    const uint8_t* base = B + size_t(sub0) * 2 * ns * rowbytes;
    brow[0] = base + size_t(nl) * rowbytes;
    brow[1] = base + size_t(ns + nl) * rowbytes;
    ncol[0] = nl;
    ncol[1] = ns + nl;
  } else {
    n0 = nt * RS_NB;
    wave_on = n0 + wave * 64 < g.N;
    const int n = min(n0 + wave * 64 + l32, g.N - 1);
    const int n1 = min(n + 32, g.N - 1);
    const size_t rowbytes = FP4 ? size_t(ns) / 2 : size_t(ns) * EBW;
    const uint8_t* base = B + size_t(ti.e) * g.n_experts_split * g.N * rowbytes;
    brow[0] = base + size_t(n) * rowbytes;
    brow[1] = base + size_t(n1) * rowbytes;
    ncol[0] = n;
    ncol[1] = n1;
  }
  // byte offset of K position k0 inside a weight row (down: plus the sub-expert stride)
  auto koff = [&](int k0) -> size_t {
    if (MODE == EPI_SWIGLU) return FP4 ? size_t(k0) / 2 : size_t(k0) * EBW;
    const size_t sub_stride = FP4 ? size_t(g.N) * ns / 2 : size_t(g.N) * ns * EBW;
    return size_t(k0 / ns) * sub_stride + (FP4 ? size_t(k0 % ns) / 2 : size_t(k0 % ns) * EBW);
  };
  // this lane's weight bytes for the stage at k0, per fragment: bf16 and fp8 64
  // contiguous bytes at 64h; MX two 16-byte pieces at 32s + 16h
  auto bsrc = [&](int f, int k0) -> const uint8_t* {
    return brow[f] + koff(k0) + (FP4 ? half * 16 : half * 64);
  };
  auto bscale_fp8 = [&](int f, int k0) -> float {
    const float* S = static_cast<const float*>(g.B_scale);
    if (MODE == EPI_SWIGLU) {
      const int rb = (f == 0 ? (n0 % ns) : ns + (n0 % ns)) / 128;
      return S[(size_t(sub0) * (2 * ns / 128) + rb) * (K / 128) + k0 / 128];
    }
    const int sub = ti.e * g.n_experts_split + k0 / ns;
    const int cb = min(n0 + wave * 64 + f * 32, g.N - 1) / 128;
    return S[(size_t(sub) * (g.N / 128) + cb) * (ns / 128) + (k0 % ns) / 128];
  };
  // fp4 weight scales of fragment f at k0: 4 scale bytes (groups k0/SG .. +3) of this
  // lane's row: MX E8M0 per 32, NVFP4 e4m3 codes per 16
  auto bscale_fp4 = [&](int f, int k0) -> uint32_t {
    const uint8_t* S = static_cast<const uint8_t*>(g.B_scale);
    if (MODE == EPI_SWIGLU)
      return *reinterpret_cast<const uint32_t*>(S + (size_t(sub0) * 2 * ns + ncol[f]) * (K / SG) + k0 / SG);
    const int sub = ti.e * g.n_experts_split + k0 / ns;
    return *reinterpret_cast<const uint32_t*>(S + (size_t(sub) * g.N + ncol[f]) * (ns / SG) + (k0 % ns) / SG);
  };

  // ---- activation copies: copy j of wave w fills LDS chunk positions (w*MS + j)*64 + lane
  const uint8_t* a_src[A_INSTR];
#pragma unroll
  for (int j = 0; j < A_INSTR; ++j) {
    const int p = (wave * A_INSTR + j) * 64 + lane, r = p >> 3, c = rs_slot(r, p & 7);
    a_src[j] = A + size_t(a_row(g, ti.row0 + min(r, ti.rows - 1))) * g.lda * EA + c * 16;
  }
  const int sa_row = ASC ? a_row(g, ti.row0 + min(tid % BM, ti.rows - 1)) : 0;
  auto load_sa = [&](int k0) -> uint32_t {        // every thread loads (rows clamped): equal vmcnt per wave
    if (MX) return *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(g.A_scale) +
                                                      size_t(sa_row) * (K / 32) + k0 / 32);
    return __float_as_uint(static_cast<const float*>(g.A_scale)[size_t(sa_row) * (K / 128) + k0 / 128]);
  };

  uint4 breg[NST][2][BCH];
  uint32_t sreg[NST];
  uint32_t sbm[NST][2];
  auto issue = [&](int k0, int buf) {
#pragma unroll
    for (int j = 0; j < A_INSTR; ++j)
      rs_copy16(a_src[j] + size_t(k0) * EA, &As[buf][(wave * A_INSTR + j) * 1024]);
    if (ASC) sreg[buf] = load_sa(k0);
    // every wave loads (inactive column waves read a clamped, valid row) so that all
    // waves count the same loads per stage
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const uint8_t* p = bsrc(f, k0);
#pragma unroll
      for (int c = 0; c < BCH; ++c) breg[buf][f][c] = *reinterpret_cast<const uint4*>(p + c * (MX ? 32 : 16));
      if (FP4) sbm[buf][f] = bscale_fp4(f, k0);
    }
  };
  constexpr int PER_STAGE = A_INSTR + (ASC ? 1 : 0) + 2 * BCH + (FP4 ? 2 : 0);   // loads per stage per thread

  f32x16 acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  // this block's K stages (a K split only in the plain store mode)
  const int nz = (MODE == EPI_STORE) ? int(gridDim.z) : 1;
  const int KT = K / KS / nz, kb = (MODE == EPI_STORE) ? int(blockIdx.z) * KT : 0;
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < KT) issue((kb + s) * KS, s);

  for (int kt0 = 0; kt0 < KT; kt0 += NST) {
#pragma unroll
    for (int buf = 0; buf < NST; ++buf) {
      const int kt = kt0 + buf;
      if (kt >= KT) break;
      // stage kt's activation copies must have landed in every wave's LDS slots;
      // the weight registers are waited for by the compiler at their first use
      if (NST >= 3 && kt + 1 < KT) rs_wait_vmcnt<(NST >= 3 ? (NST - 2) * PER_STAGE : 0)>();
      else rs_wait_vmcnt<0>();
      if (!BF16 && tid < BM) Sa[buf][tid] = sreg[buf];
      __syncthreads();
      const int nb = (buf + NST - 1) % NST;
      if (kt + NST - 1 < KT) issue((kb + kt + NST - 1) * KS, nb);
      if (!wave_on) continue;
      const uint8_t* Ab = As[buf];
      if (BF16) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 b0 = __builtin_bit_cast(bf16x8, breg[buf][0][s]);
          const bf16x8 b1 = __builtin_bit_cast(bf16x8, breg[buf][1][s]);
#pragma unroll
          for (int i = 0; i < MS; ++i) {
            if (i < act_ms) {
              const bf16x8 a =
                  __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Ab + rs_swz(i * 32 + l32, half * 4 + s)));
              acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[i][0], 0, 0, 0);
              acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[i][1], 0, 0, 0);
            }
          }
        }
      } else if (NV) {
        // fp16 MFMA on exactly dequantised operands: the activations are fp16 values
        // already; the weights' e2m1 codes become fp16 by a byte lookup, times the
        // group's e4m3 scale (every product is exact in fp16).  Lane half h, step s
        // takes k = 32h + 8s .. +8 on both sides: step s uses dword s of the lane's
        // 16 weight bytes and scale byte 2h + s/2 of the stage's four.
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          f16x8 bw[2];
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const uint32_t w = (s == 0) ? breg[buf][f][0].x : (s == 1) ? breg[buf][f][0].y
                             : (s == 2) ? breg[buf][f][0].z : breg[buf][f][0].w;
            const _Float16 sc = _Float16(e4m3_to_f32((sbm[buf][f] >> (8 * (2 * half + (s >> 1)))) & 0xffu));
            bw[f] = e2m1x8_to_f16(w, f16x2{sc, sc});
          }
#pragma unroll
          for (int i = 0; i < MS; ++i) {
            if (i < act_ms) {
              const f16x8 a =
                  __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(Ab + rs_swz(i * 32 + l32, half * 4 + s)));
              acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bw[0], a, acc[i][0], 0, 0, 0);
              acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bw[1], a, acc[i][1], 0, 0, 0);
            }
          }
        }
      } else if (FP8) {
        const float sb0 = bscale_fp8(0, (kb + kt) * KS), sb1 = bscale_fp8(1, (kb + kt) * KS);
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          if (i >= act_ms) continue;
          const int ar = i * 32 + l32;
          i32x8 a[2];
#pragma unroll
          for (int s = 0; s < 2; ++s)
            a[s] = rs_cat(*reinterpret_cast<const uint4*>(Ab + rs_swz(ar, 4 * half + 2 * s)),
                          *reinterpret_cast<const uint4*>(Ab + rs_swz(ar, 4 * half + 2 * s + 1)));
          const float ra = __uint_as_float(Sa[buf][ar]);   // this lane's token row
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            f32x16 part;
#pragma unroll
            for (int r = 0; r < 16; ++r) part[r] = 0.0f;
#pragma unroll
            for (int s = 0; s < 2; ++s)
              part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  rs_cat(breg[buf][f][2 * s], breg[buf][f][2 * s + 1]), a[s], part, 0, 0, 0, 127, 0, 127);
            const float rs = ra * (f ? sb1 : sb0);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][f][r] = fmaf(part[r], rs, acc[i][f][r]);
          }
        }
      } else {  // MX
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          if (i >= act_ms) continue;
          const int ar = i * 32 + l32;
          const uint32_t sa4 = Sa[buf][ar];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            // K 64s + 16h .. +16 and 64s + 32 + 16h .. +16 of the stage
            const i32x8 a = rs_cat(*reinterpret_cast<const uint4*>(Ab + rs_swz(ar, 4 * s + half)),
                                   *reinterpret_cast<const uint4*>(Ab + rs_swz(ar, 4 * s + 2 + half)));
            const int sh = 8 * (2 * s + half);
            const int sa = int((sa4 >> sh) & 0xffu);
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const uint4 bw = breg[buf][f][s];
              const i32x8 b = i32x8{int(bw.x), int(bw.y), int(bw.z), int(bw.w), 0, 0, 0, 0};
              acc[i][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  b, a, acc[i][f], 4, 0, 0, int((sbm[buf][f] >> sh) & 0xffu), 0, sa);
            }
          }
        }
      }
    }
  }

  // ---- epilogues.  bf16: lane l, register r of row block i holds token row
  // i*32 + acc_row(r, l) and column l & 31 of the fragment (measured faster for
  // decode).  fp8 and MX: the weight fragment is the MFMA's first operand, so lane
  // l, register r = 4q + e holds token row i*32 + (l & 31) and column
  // 8q + 4*(l>>5) + e, and each lane stores runs of four columns.
  auto pack_bf16 = [](float a, float b, float c, float d) {
    return uint2{uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16),
                 uint32_t(f32_to_bf16(c)) | (uint32_t(f32_to_bf16(d)) << 16)};
  };
  if (MODE == EPI_SWIGLU) {
    const int c0 = n0 + wave * 32 + 4 * half;      // h column of register 0
    if (BF16) {
      uint16_t* Hh = static_cast<uint16_t*>(g.out);
      const int col = n0 + wave * 32 + l32;
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        if (i >= act_ms) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + acc_row(r, lane);
          if (row < ti.rows) Hh[size_t(ti.row0 + row) * g.ldo + col] = f32_to_bf16(swiglu_f32(acc[i][0][r], acc[i][1][r], g.swiglu_limit));
        }
      }
    } else if (MX) {                               // MXFP8 per (row, 32 columns): one fragment per block
      uint8_t* Hq = static_cast<uint8_t*>(g.out);
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        if (i >= act_ms) continue;
        float hv[16], m = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          hv[r] = swiglu_f32(acc[i][0][r], acc[i][1][r], g.swiglu_limit);
          m = fmaxf(m, fabsf(hv[r]));
        }
        m = fmaxf(m, __shfl_xor(m, 32, 64));       // the row's other 16 columns
        const int e = mx_exponent_e4m3(m);
        const float inv = exp2i(-e);
        const int row = i * 32 + l32;
        if (row < ti.rows) {
          uint8_t* hrow = Hq + size_t(ti.row0 + row) * g.ldo + c0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t packed = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) packed |= f32_to_e4m3(hv[4 * q + k] * inv) << (8 * k);
            *reinterpret_cast<uint32_t*>(hrow + 8 * q) = packed;
          }
          if (half == 0)
            static_cast<uint8_t*>(g.out_scale)[size_t(ti.row0 + row) * (g.N / 32) + (n0 + wave * 32) / 32] =
                uint8_t(e + 127);
        }
      }
    } else if (NV) {                               // NVFP4 per (row, 16 columns), stored as fp16 values
      uint16_t* Hf = static_cast<uint16_t*>(g.out);
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        if (i >= act_ms) continue;
        float hv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) hv[r] = swiglu_f32(acc[i][0][r], acc[i][1][r], g.swiglu_limit);
        // group j (columns 16j .. 16j+15) = registers 8j .. 8j+7 of both lane halves
        float sc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float m = 0.0f;
#pragma unroll
          for (int r = 8 * j; r < 8 * j + 8; ++r) m = fmaxf(m, fabsf(hv[r]));
          sc[j] = nvfp4_scale(fmaxf(m, __shfl_xor(m, 32, 64)));
        }
        const int row = i * 32 + l32;
        if (row < ti.rows) {
          uint16_t* hrow = Hf + size_t(ti.row0 + row) * g.ldo + c0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float s = sc[q >> 1];
            const f16x2 lo = {_Float16(nvfp4_value(hv[4 * q], s)), _Float16(nvfp4_value(hv[4 * q + 1], s))};
            const f16x2 hi = {_Float16(nvfp4_value(hv[4 * q + 2], s)), _Float16(nvfp4_value(hv[4 * q + 3], s))};
            *reinterpret_cast<uint2*>(hrow + 8 * q) = uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          }
        }
      }
    } else {                                       // fp8 per (row, 128 columns): across the four waves
      uint8_t* Hq = static_cast<uint8_t*>(g.out);
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        if (i >= act_ms) continue;                 // uniform across the block
        float hv[16], m = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          hv[r] = swiglu_f32(acc[i][0][r], acc[i][1][r], g.swiglu_limit);
          m = fmaxf(m, fabsf(hv[r]));
        }
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const int row = i * 32 + l32;
        if (half == 0) amax_lds[wave][row] = m;
        __syncthreads();
        const float amax = fmaxf(fmaxf(amax_lds[0][row], amax_lds[1][row]), fmaxf(amax_lds[2][row], amax_lds[3][row]));
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        if (row < ti.rows) {
          uint8_t* hrow = Hq + size_t(ti.row0 + row) * g.ldo + c0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t packed = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) packed |= f32_to_e4m3(hv[4 * q + k] / sc) << (8 * k);
            *reinterpret_cast<uint32_t*>(hrow + 8 * q) = packed;
          }
          if (wave == 0 && half == 0)
            static_cast<float*>(g.out_scale)[size_t(ti.row0 + row) * (g.N / 128) + n0 / 128] = sc;
        }
        __syncthreads();
      }
    }
  } else if (BF16) {
    if (!wave_on) return;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int col = n0 + wave * 64 + f * 32 + l32;
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        if (i >= act_ms) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + acc_row(r, lane);
          if (row >= ti.rows) continue;
          const size_t o = size_t(ti.row0 + row) * g.ldo + col;
          if (g.out_f32) static_cast<float*>(g.out)[blockIdx.z * g.split_stride + o] = acc[i][f][r];
          else static_cast<uint16_t*>(g.out)[o] = f32_to_bf16(acc[i][f][r]);
        }
      }
    }
  } else {
    if (!wave_on) return;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int c0 = n0 + wave * 64 + f * 32 + 4 * half;
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int row = i * 32 + l32;
        if (i >= act_ms || row >= ti.rows) continue;
        const size_t o = size_t(ti.row0 + row) * g.ldo + c0;
        const f32x16& a = acc[i][f];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (g.out_f32)
            *reinterpret_cast<float4*>(static_cast<float*>(g.out) + blockIdx.z * g.split_stride + o + 8 * q) =
                float4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
          else
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + o + 8 * q) =
                pack_bf16(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        }
      }
    }
  }
}

// Register-ring depth of the weight stream (stages; NST-1 in flight per wave).
constexpr int RS_NST1 = 2, RS_NST2 = 3;

template <int MODE, int RECIPE>
static void rs_launch(int ms, dim3 grid, const GemmArgs& g, hipStream_t st) {
  if constexpr (RECIPE != MOE_RECIPE_FP8_B128) {
    if (ms >= 4) {                                 // 128-row tiles, held to two waves per SIMD
      ffn_rs_kernel<4, MODE, RECIPE, 2, 2><<<grid, 256, 0, st>>>(g);
      return;
    }
  }
  // NVFP4 moves 0.56 weight bytes per element: a deeper ring keeps enough of them in flight
  if (ms <= 1) ffn_rs_kernel<1, MODE, RECIPE, (RECIPE == MOE_RECIPE_NVFP4 ? 6 : RS_NST1)><<<grid, 256, 0, st>>>(g);
  else ffn_rs_kernel<2, MODE, RECIPE, RS_NST2, (RECIPE == MOE_RECIPE_FP8_B128 ? 2 : 1)><<<grid, 256, 0, st>>>(g);
}

template <int MODE>
static hipError_t rs_launch_recipe(int recipe, int ms, dim3 grid, const GemmArgs& g, hipStream_t st) {
  if (recipe == MOE_RECIPE_BF16) rs_launch<MODE, MOE_RECIPE_BF16>(ms, grid, g, st);
  else if (recipe == MOE_RECIPE_FP8_B128) rs_launch<MODE, MOE_RECIPE_FP8_B128>(ms, grid, g, st);
  else if (recipe == MOE_RECIPE_NVFP4) rs_launch<MODE, MOE_RECIPE_NVFP4>(ms, grid, g, st);
  else rs_launch<MODE, MOE_RECIPE_MXFP4>(ms, grid, g, st);
  return hipGetLastError();
}

// Tiles of ms*32 rows (ms = 1 or 2; bf16, MXFP4 and NVFP4 also 4).  bf16 is used for the shared experts of every
// bf16-activation recipe as well.
hipError_t launch_rs_swiglu(int recipe, int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  return rs_launch_recipe<EPI_SWIGLU>(recipe, ms, dim3(g.N / 128, m_tiles), g, st);
}
// ksplit > 1: fp32 partial products of ksplit equal K ranges (K / 64 / ksplit stages
// each, an integer), see GemmArgs::split_stride.
hipError_t launch_rs_down(int recipe, int ms, int m_tiles, const GemmArgs& g, hipStream_t st, int ksplit) {
  return rs_launch_recipe<EPI_STORE>(recipe, ms, dim3((g.N + RS_NB - 1) / RS_NB, m_tiles, ksplit), g, st);
}

}  // namespace moe
