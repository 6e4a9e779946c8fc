// Grouped expert GEMMs for prefill-sized expert blocks (moe_infer's per-expert
// gate/up/down + SiLU over contiguous row blocks: DeepSeek-V3 walk-through,
// pwwt.cn/news/5781524, section 3.4), bf16 and fp8 (128x128 block scales).
//
// Tile: up to 32*MS rows x 256 weight rows (SwiGLU: 128 gate_proj rows and the
// matching 128 up_proj rows; down: 256 output columns) on a WM x WN grid of
// wavefronts.  Wave (wm, wn) owns the 32-row MFMA fragments wm, wm+WM, wm+2WM,
// ... and 8/WN of the eight 32-wide weight fragments (SwiGLU: 4/WN gate fragments
// and the matching up fragments, so that SiLU(g)*u pairs sit in the same lane and
// register).  A partial tile (the last rows of an expert) skips the same share of
// row fragments in every wave and costs time in proportion to its rows.
//
// Both operands are staged through LDS with gfx950's direct global->LDS 16-byte
// loads (global_load_lds_dwordx4) into a ring of NST stages of ROWB-byte rows
// (ROWB/2 bf16 or ROWB fp8 of K per stage).  The 16-byte chunk c of LDS row r sits
// at slot c ^ g(r), with g(r) = ((r>>1) ^ (r>>2)) & 3 for 64-byte rows and
// (r ^ (r>>1)) & 7 for 128-byte rows: any 16 consecutive rows reading one chunk hit
// 16 distinct 16-byte slots of a 256-byte bank window (and any 8 rows, 8 distinct
// slots of a 128-byte window).  The XOR is applied on the global side, so the LDS
// writes of one copy instruction (64 lanes x 16 bytes) stay contiguous as the
// hardware requires.  128-byte rows take whole cache lines per stage.
//
// Tiles are numbered (row tile, column tile), column tile fastest, and mapped so
// that consecutive numbers run on the same XCD: column tiles sharing an
// activation block, and the row tiles of one expert sharing weight rows, meet in
// that XCD's L2.
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int NB = 256;          // weight rows per tile

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Slot of logical 16-byte chunk c in LDS row r (rows of ROWB bytes).  For 64-byte rows
// g(r) = ((r>>1) ^ (r>>2)) & 3, for 128-byte rows g(r) = (r ^ (r>>1)) & 7: in both
// cases any 16 consecutive rows reading one chunk land on 16 distinct 16-byte slots
// of a 256-byte bank window, and any 8 rows on 8 distinct slots of a 128-byte one.
template <int ROWB>
__device__ __forceinline__ int swz_slot(int r, int c) {
  if (ROWB == 64) return c ^ (((r >> 1) ^ (r >> 2)) & 3);
  return c ^ ((r ^ (r >> 1)) & 7);
}
template <int ROWB>
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + (swz_slot<ROWB>(r, c) << 4); }

__device__ __forceinline__ void async_copy16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// s_waitcnt with vmcnt = n, other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Bijective map of a linear block index b < V to a tile number so that the blocks
// one XCD runs (b % 8 fixed) cover a contiguous range of tile numbers.
__device__ __forceinline__ int xcd_tile(int b, int V) {
  const int q = V >> 3, r = V & 7, x = b & 7, l = b >> 3;
  return (x < r) ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
}

enum Kind { KIND_BF16 = 0, KIND_FP8 = 1 };

__device__ __forceinline__ i32x8 cat(uint4 lo, uint4 hi) {
  return i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

}  // namespace

// Every LDS row a wave reads is 32*m + l32 for its lane's l32, so its swizzle key
// is that of l32: a fragment's operand sits at a constant offset from the wave's
// base plus one per-lane offset per chunk.  Row offset of weight fragment f within
// a wave's share: SwiGLU (SPLIT = gate fragments per wave) interleaves the gate
// half (rows 0..127) and the up half (rows 128..255).
template <int SPLIT>
__device__ constexpr int bfrag_row(int f) { return SPLIT > 0 ? (f < SPLIT ? 0 : 128) + (f % SPLIT) * 32 : f * 32; }

// One stage (ROWB/2 K of bf16) for the NJ row fragments of this wave that hold
// real rows: every LDS operand read of the stage is issued before its MFMAs, with
// no branch in between, so the reads overlap the matrix pipeline.
template <int NJ, int MW, int NF, int WM, int ROWB, int SPLIT>
__device__ __forceinline__ void stage_bf16(f32x16 (&acc)[MW][NF], const uint8_t* Aw, const uint8_t* Bw, int l32,
                                           int half) {
  constexpr int NS = ROWB / 32;                        // 16-deep MFMA steps per stage
  bf16x8 bv[NS][NF], av[NS][NJ];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int off = l32 * ROWB + (swz_slot<ROWB>(l32, 2 * s + half) << 4);   // k = 16s + 8h .. +8
#pragma unroll
    for (int f = 0; f < NF; ++f)
      bv[s][f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Bw + bfrag_row<SPLIT>(f) * ROWB + off));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      av[s][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Aw + WM * 32 * ROWB * j + off));
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[j][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[s][j], bv[s][f], acc[j][f], 0, 0, 0);
}

// One stage (ROWB K of fp8) with the 128x128-block scales: the MFMA runs with unit
// scales (lane half h takes bytes 64s + 32h .. +32 of the row at sub-step s) and
// each fragment's partial sum is scaled by a_scale[row] * b_scale[block]; a stage
// never straddles a 128-block.  Sw: this wave's row scales (its fragment 0 first).
template <int NJ, int MW, int NF, int WM, int ROWB, int SPLIT>
__device__ __forceinline__ void stage_fp8(f32x16 (&acc)[MW][NF], const uint8_t* Aw, const uint8_t* Bw,
                                          const float* Sw, const float (&sb)[NF], int l32, int half) {
  constexpr int NS = ROWB / 64;
  int off[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int q = 0; q < 2; ++q) off[s][q] = l32 * ROWB + (swz_slot<ROWB>(l32, 4 * s + 2 * half + q) << 4);
  i32x8 bv[NS][NF];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint8_t* p = Bw + bfrag_row<SPLIT>(f) * ROWB;
      bv[s][f] = cat(*reinterpret_cast<const uint4*>(p + off[s][0]), *reinterpret_cast<const uint4*>(p + off[s][1]));
    }
  // one row fragment at a time: its operands and row scales live only for its MFMAs
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint8_t* p = Aw + WM * 32 * ROWB * j;
    i32x8 av[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
      av[s] = cat(*reinterpret_cast<const uint4*>(p + off[s][0]), *reinterpret_cast<const uint4*>(p + off[s][1]));
    float ra[16];                                     // rows 8q + 4h + 0..3 of the fragment
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(Sw + WM * 32 * j + 8 * q + 4 * half);
      ra[4 * q] = v.x; ra[4 * q + 1] = v.y; ra[4 * q + 2] = v.z; ra[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      f32x16 part;
#pragma unroll
      for (int r = 0; r < 16; ++r) part[r] = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[s], bv[s][f], part, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][f][r] += part[r] * (ra[r] * sb[f]);
    }
  }
}

// MS: 32-row fragments per tile; WM x WN: wavefront grid; ROWB: bytes of K per
// LDS row and stage (64 or 128); NST: stages in the LDS ring.
template <int MS, int MODE, int KIND, int WM, int WN, int ROWB, int NST>
__global__ __launch_bounds__(64 * WM * WN, 1) void ffn_lds_kernel(GemmArgs g) {
  constexpr int NW = WM * WN;                       // wavefronts
  constexpr int BM = MS * 32;
  constexpr int MW = MS / WM;                       // row fragments per wave
  constexpr int NF = 8 / WN;                        // weight fragments per wave
  constexpr int NFG = NF / 2;                       // SwiGLU: gate (= up) fragments per wave
  constexpr int A_INSTR = BM * (ROWB / 16) / 64 / NW;   // async copies per wave per stage (A)
  constexpr int B_INSTR = NB * (ROWB / 16) / 64 / NW;   // (B)
  static_assert(MW >= 1 && NFG >= 1 && A_INSTR >= 1 && B_INSTR >= 1, "tile shape");
  static_assert(MS * 32 * (ROWB / 16) == A_INSTR * 64 * NW, "A copies cover the stage");
  constexpr int EB = (KIND == KIND_BF16) ? 2 : 1;   // bytes per element
  constexpr int KS = ROWB / EB;                     // K per stage
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  uint8_t* As = smem;                               // [NST][BM * ROWB]
  uint8_t* Bs = smem + NST * BM * ROWB;             // [NST][NB * ROWB]
  float* Sa = reinterpret_cast<float*>(Bs + NST * NB * ROWB);   // fp8: [NST][BM] row scales
  float* amax_lds = Sa + NST * BM;                               // fp8 epilogue: [WN][BM]

  const int ncols = (MODE == EPI_SWIGLU) ? g.N / 128 : (g.N + NB - 1) / NB;
  const int ntiles_m = g.tiles ? g.tiles[0] : (g.dense_rows + BM - 1) / BM;
  const int V = ncols * ntiles_m;
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  if (b >= V) return;
  const int tnum = xcd_tile(b, V);
  const int mt = tnum / ncols, nt = tnum - mt * ncols;
  TileInfo ti;
  if (g.tiles) {
    ti.e = g.tiles[1 + 2 * mt];
    ti.row0 = g.offsets[ti.e] + g.tiles[2 + 2 * mt];
    ti.rows = min(BM, g.offsets[ti.e + 1] - ti.row0);
  } else {
    ti.e = 0;
    ti.row0 = mt * BM;
    ti.rows = min(BM, g.dense_rows - ti.row0);
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave % WM, wn = wave / WM;
  const int K = g.K, ns = g.nsplit;
  const uint8_t* A = static_cast<const uint8_t*>(g.A);
  const uint8_t* B = static_cast<const uint8_t*>(g.B);
  const int act_ms = (ti.rows + 31) >> 5;           // 32-row fragments holding real rows

  // ---- global sources of this thread's async copies: copy j of wave w fills LDS
  // chunk positions p = (w*INSTR + j)*64 + lane -> row p / (ROWB/16), slot
  // p % (ROWB/16), logical chunk slot ^ g(row)
  const uint8_t* a_src[A_INSTR];
#pragma unroll
  for (int j = 0; j < A_INSTR; ++j) {
    const int p = (wave * A_INSTR + j) * 64 + lane, r = p / (ROWB / 16);
    const int c = swz_slot<ROWB>(r, p % (ROWB / 16));
    const int row = ti.row0 + min(r, ti.rows - 1);
    a_src[j] = A + (size_t(row) * g.lda) * EB + c * 16;
  }
  int n0, sub0 = 0;
  if (MODE == EPI_SWIGLU) {
    n0 = nt * 128;
    sub0 = ti.e * g.n_experts_split + n0 / ns;
  } else {
    n0 = nt * NB;
  }
  const uint8_t* b_src[B_INSTR];
#pragma unroll
  for (int j = 0; j < B_INSTR; ++j) {
    const int p = (wave * B_INSTR + j) * 64 + lane, r = p / (ROWB / 16);
    const int c = swz_slot<ROWB>(r, p % (ROWB / 16));
    size_t rowoff;
    if (MODE == EPI_SWIGLU) {
      const int wr = (r < 128) ? (n0 % ns + r) : (ns + n0 % ns + r - 128);
      rowoff = (size_t(sub0) * 2 * ns + wr) * size_t(K);
    } else {
      const int n = min(n0 + r, g.N - 1);
      rowoff = size_t(ti.e) * g.n_experts_split * g.N * ns + size_t(n) * ns;
    }
    b_src[j] = B + rowoff * EB + c * 16;
  }
  auto koff_bytes = [&](int k0) -> size_t {
    if (MODE == EPI_SWIGLU) return size_t(k0) * EB;
    return (size_t(k0 / ns) * g.N * ns + (k0 % ns)) * EB;
  };
  auto issue = [&](int k0, int buf) {
#pragma unroll
    for (int j = 0; j < A_INSTR; ++j)
      async_copy16(a_src[j] + size_t(k0) * EB, As + buf * BM * ROWB + (wave * A_INSTR + j) * 1024);
    const size_t ko = koff_bytes(k0);
#pragma unroll
    for (int j = 0; j < B_INSTR; ++j) async_copy16(b_src[j] + ko, Bs + buf * NB * ROWB + (wave * B_INSTR + j) * 1024);
  };
  // fp8 activation scale of row (tid % BM) for the 128-block holding k0.  Every
  // thread loads (rows clamped) so that all waves count the same loads in flight.
  auto load_sa = [&](int k0) -> float {
    const float* S = static_cast<const float*>(g.A_scale);
    const int r = min(tid % BM, ti.rows - 1);
    return S[size_t(ti.row0 + r) * (K / 128) + k0 / 128];
  };
  // Tile-relative weight column of each of this wave's fragments (SwiGLU: the h
  // column block of the gate/up pair); the wave's first LDS weight row.
  constexpr int SPLIT = (MODE == EPI_SWIGLU) ? NFG : 0;
  int fcol[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) fcol[f] = (MODE == EPI_SWIGLU) ? (wn * NFG + f % NFG) * 32 : (wn * NF + f) * 32;
  const int brow0 = (MODE == EPI_SWIGLU) ? wn * NFG * 32 : wn * NF * 32;
  // fp8 weight scale of this wave's fragment f at k0 (uniform across the wave)
  auto bscale_fp8 = [&](int f, int k0) -> float {
    const float* S = static_cast<const float*>(g.B_scale);
    if (MODE == EPI_SWIGLU) {
      const int rb = ((f < NFG) ? (n0 % ns) : ns + (n0 % ns)) / 128;
      return S[(size_t(sub0) * (2 * ns / 128) + rb) * (K / 128) + k0 / 128];
    }
    const int sub = ti.e * g.n_experts_split + k0 / ns;
    const int cb = min(n0 + fcol[f], g.N - 1) / 128;
    return S[(size_t(sub) * (g.N / 128) + cb) * (ns / 128) + (k0 % ns) / 128];
  };

  f32x16 acc[MW][NF];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  const int KT = K / KS;
  constexpr int PER_STAGE = A_INSTR + B_INSTR + (KIND == KIND_FP8 ? 1 : 0);   // loads per thread per stage
  float sa_reg[NST];
  // prologue: stages 0 .. NST-2 in flight
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    if (s < KT) {
      issue(s * KS, s);
      if (KIND == KIND_FP8) sa_reg[s] = load_sa(s * KS);
    }
  }
  // row fragments of this wave that hold real rows (wave-uniform)
  const int nj = min(MW, max(0, (act_ms - wm + WM - 1) / WM));
  auto compute = [&](int kt, int buf) {
    const uint8_t* Aw = As + buf * BM * ROWB + wm * 32 * ROWB;
    const uint8_t* Bw = Bs + buf * NB * ROWB + brow0 * ROWB;
    if (KIND == KIND_BF16) {
      if (MW >= 4 && nj == 4) stage_bf16<(MW >= 4 ? 4 : 1), MW, NF, WM, ROWB, SPLIT>(acc, Aw, Bw, l32, half);
      else if (MW >= 3 && nj == 3) stage_bf16<(MW >= 3 ? 3 : 1), MW, NF, WM, ROWB, SPLIT>(acc, Aw, Bw, l32, half);
      else if (MW >= 2 && nj == 2) stage_bf16<(MW >= 2 ? 2 : 1), MW, NF, WM, ROWB, SPLIT>(acc, Aw, Bw, l32, half);
      else if (nj == 1) stage_bf16<1, MW, NF, WM, ROWB, SPLIT>(acc, Aw, Bw, l32, half);
    } else {
      float sb[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) sb[f] = bscale_fp8(f, kt * KS);
      const float* Sw = Sa + buf * BM + wm * 32;
      if (MW >= 4 && nj == 4) stage_fp8<(MW >= 4 ? 4 : 1), MW, NF, WM, ROWB, SPLIT>(acc, Aw, Bw, Sw, sb, l32, half);
      else if (MW >= 3 && nj == 3) stage_fp8<(MW >= 3 ? 3 : 1), MW, NF, WM, ROWB, SPLIT>(acc, Aw, Bw, Sw, sb, l32, half);
      else if (MW >= 2 && nj == 2) stage_fp8<(MW >= 2 ? 2 : 1), MW, NF, WM, ROWB, SPLIT>(acc, Aw, Bw, Sw, sb, l32, half);
      else if (nj == 1) stage_fp8<1, MW, NF, WM, ROWB, SPLIT>(acc, Aw, Bw, Sw, sb, l32, half);
    }
  };
  for (int kt0 = 0; kt0 < KT; kt0 += NST) {
#pragma unroll
    for (int buf = 0; buf < NST; ++buf) {            // unrolled: the ring slot is a constant
      const int kt = kt0 + buf;
      if (kt >= KT) break;
      // wait until stage kt has landed (later stages may still be in flight)
      const int ahead = min(NST - 2, KT - 1 - kt);
      if (NST >= 4 && ahead >= 2) wait_vmcnt<(NST >= 4 ? 2 : 0) * PER_STAGE>();
      else if (NST >= 3 && ahead >= 1) wait_vmcnt<PER_STAGE>();
      else wait_vmcnt<0>();
      if (KIND == KIND_FP8 && tid < BM) Sa[buf * BM + tid] = sa_reg[buf];
      __syncthreads();
      // refill the slot consumed in the previous iteration
      const int nb = (buf + NST - 1) % NST;
      if (kt + NST - 1 < KT) {
        issue((kt + NST - 1) * KS, nb);
        if (KIND == KIND_FP8) sa_reg[nb] = load_sa((kt + NST - 1) * KS);
      }
      compute(kt, buf);
    }
  }

  // ---- epilogues
  if (MODE == EPI_SWIGLU) {
    if (KIND == KIND_BF16) {
      uint16_t* Hh = static_cast<uint16_t*>(g.out);
#pragma unroll
      for (int j = 0; j < MW; ++j) {
        const int i = wm + WM * j;
        if (i >= act_ms) continue;
#pragma unroll
        for (int f = 0; f < NFG; ++f) {
          const int col = n0 + fcol[f] + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + acc_row(r, lane);
            if (row < ti.rows)
              Hh[size_t(ti.row0 + row) * g.ldo + col] = f32_to_bf16(silu_f32(acc[j][f][r]) * acc[j][f + NFG][r]);
          }
        }
      }
    } else {
      // h re-quantised per (row, 128 columns): the tile's 128 h columns are one block,
      // split over the WN column waves
      uint8_t* Hq = static_cast<uint8_t*>(g.out);
#pragma unroll
      for (int j = 0; j < MW; ++j) {
        const int i = wm + WM * j;
        const bool on = i < act_ms;
        float hv[NFG][16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float m = 0.0f;
#pragma unroll
          for (int f = 0; f < NFG; ++f) {
            hv[f][r] = silu_f32(acc[j][f][r]) * acc[j][f + NFG][r];
            m = fmaxf(m, fabsf(hv[f][r]));
          }
          m = max_over_lanes32(m);
          if (on && l32 == 0) amax_lds[wn * BM + i * 32 + acc_row(r, lane)] = m;
        }
        __syncthreads();
        if (on) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + acc_row(r, lane);
            float amax = amax_lds[row];
#pragma unroll
            for (int q = 1; q < WN; ++q) amax = fmaxf(amax, amax_lds[q * BM + row]);
            const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            if (row < ti.rows) {
#pragma unroll
              for (int f = 0; f < NFG; ++f)
                Hq[size_t(ti.row0 + row) * g.ldo + n0 + fcol[f] + l32] = uint8_t(f32_to_e4m3(hv[f][r] / s));
              if (wn == 0 && l32 == 0)
                static_cast<float*>(g.out_scale)[size_t(ti.row0 + row) * (g.N / 128) + n0 / 128] = s;
            }
          }
        }
        __syncthreads();
      }
    }
  } else {  // EPI_STORE: bf16 y rows, or fp32 rows (out_f32)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int col = n0 + fcol[f] + l32;
      if (n0 + fcol[f] >= g.N) continue;               // partial column tile (g.N % 128 == 0)
#pragma unroll
      for (int j = 0; j < MW; ++j) {
        const int i = wm + WM * j;
        if (i >= act_ms) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + acc_row(r, lane);
          if (row >= ti.rows) continue;
          const size_t o = size_t(ti.row0 + row) * g.ldo + col;
          if (g.out_f32) static_cast<float*>(g.out)[o] = acc[j][f][r];
          else static_cast<uint16_t*>(g.out)[o] = f32_to_bf16(acc[j][f][r]);
        }
      }
    }
  }
}

template <int MS, int WN, int ROWB, int NST>
constexpr size_t lds_smem_bytes() {
  return size_t(NST) * (MS * 32 + NB) * ROWB + size_t(NST + WN) * MS * 32 * 4;
}

template <int MS, int MODE, int KIND, int WM, int WN, int ROWB, int NST>
void launch_lds_variant(dim3 grid, const GemmArgs& g, hipStream_t st) {
  constexpr size_t smem = lds_smem_bytes<MS, WN, ROWB, NST>();
  static_assert(smem <= 160 * 1024, "LDS budget");
  auto kfn = ffn_lds_kernel<MS, MODE, KIND, WM, WN, ROWB, NST>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kfn), hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
  kfn<<<grid, 64 * WM * WN, smem, st>>>(g);
}

// Production configurations, 128-byte rows in a two-stage ring.  bf16: 2 x 2
// wavefronts, up to 256-row tiles (the accumulators stay in the MFMA's own
// registers).  fp8: 2 x 4 wavefronts (two per SIMD), so that 256-row tiles fit:
// the block-scale FMAs keep the accumulators in ordinary VGPRs.
template <int MODE, int KIND>
static hipError_t launch_lds_ms(int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  const int ncols = (MODE == EPI_SWIGLU) ? g.N / 128 : (g.N + NB - 1) / NB;
  const dim3 grid(ncols, m_tiles);
  if constexpr (KIND == KIND_FP8) {
    if (ms <= 4) launch_lds_variant<4, MODE, KIND, 2, 4, 128, 2>(grid, g, st);
    else launch_lds_variant<8, MODE, KIND, 2, 4, 128, 2>(grid, g, st);
  } else {
    if (ms <= 2) launch_lds_variant<2, MODE, KIND, 2, 2, 128, 2>(grid, g, st);
    else if (ms <= 4) launch_lds_variant<4, MODE, KIND, 2, 2, 128, 2>(grid, g, st);
    else launch_lds_variant<8, MODE, KIND, 2, 2, 128, 2>(grid, g, st);
  }
  return hipGetLastError();
}

hipError_t launch_lds_swiglu(bool fp8, int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  return fp8 ? launch_lds_ms<EPI_SWIGLU, KIND_FP8>(ms, m_tiles, g, st)
             : launch_lds_ms<EPI_SWIGLU, KIND_BF16>(ms, m_tiles, g, st);
}
hipError_t launch_lds_down(bool fp8, int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  return fp8 ? launch_lds_ms<EPI_STORE, KIND_FP8>(ms, m_tiles, g, st)
             : launch_lds_ms<EPI_STORE, KIND_BF16>(ms, m_tiles, g, st);
}

}  // namespace moe
