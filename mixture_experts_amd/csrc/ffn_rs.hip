// Grouped expert GEMMs for experts with few rows (decode, fine-grained and the long
// tail of a skewed load): moe_infer's per-expert gate/up/down + SiLU
// (DeepSeek-V3 walk-through, pwwt.cn/news/5781524, section 3.4) where the time
// goes into streaming each expert's weights once from HBM.
//
// Tile: 32*MS rows x 256 weight rows (SwiGLU: 128 gate_proj + the matching 128
// up_proj rows; down: 256 output columns); four wavefronts, wave w owns every row
// and weight rows [32w, 32w+32) of each half.  Weights go straight from HBM into
// MFMA B-operand registers through a ring of NST register stages (NST-1 stages in
// flight per wave), each lane reading its half of the row's 128 bytes per stage
// (MXFP4 down GEMM: 64) as contiguous 16-byte loads;
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
//             scales on both operands, K = 256 per stage (128 weight bytes per
//             row: one full cache line); 128 in the down GEMM.  Operand layout measured on gfx950: an
//             fp8 operand lane (half h) holds K = 16h + 0..15 and 32 + 16h + 0..15,
//             an fp4 operand lane holds K = 32h + 0..31 (even K in the low
//             nibble), and the scale of lane (row, h) applies to K block h.  MFMA
//             m of a stage gives weight lane half h the stage's K (KS/2)h + 32m
//             .. +32.
//   nvfp4     v_mfma_f32_32x32x16_f16 on exactly dequantised operands, K = 256 per
//             stage: activations arrive as the fp16 values of their NVFP4
//             quantisation; e2m1 weights are turned into fp16 in registers (byte
//             lookup of the fp16 high byte, times the group's e4m3 scale: every
//             such product is exact in fp16).  Step s gives lane half h the
//             stage's K 128h + 8s .. +8.
// The fp4 stages are twice (MX) or four times (NVFP4) as deep as the bf16 one so
// that every stage still reads whole 128-byte lines of each weight row: a stage
// that reads part of a line leaves the rest to a later stage, by when the line
// has left L2 and is fetched again.
// The SwiGLU output h is written as bf16, or re-quantised to the activation format
// (NVFP4: stored as fp16 values).
#include <algorithm>
#include <type_traits>

#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int RS_ROWB = 128;     // bf16 / fp8: activation bytes of K per LDS row and stage
constexpr int RS_NB = 256;       // weight rows per tile

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Slot of logical 16-byte chunk c in an LDS row r of ROWB bytes: rows of 128 bytes
// share a bank line in pairs; longer rows start every bank line afresh.
template <int ROWB>
__device__ __forceinline__ int rs_slot(int r, int c) {
  return ROWB == 128 ? c ^ ((r ^ (r >> 1)) & 7) : c ^ (r & 15);
}
template <int ROWB>
__device__ __forceinline__ int rs_swz(int r, int c) { return r * ROWB + (rs_slot<ROWB>(r, c) << 4); }

template <int N>
__device__ __forceinline__ void rs_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Workgroup barrier that leaves the weight loads into registers in flight.  A
// fenced barrier (__syncthreads(), or a release fence on LDS alone while async
// LDS copies are outstanding) waits for every vector memory operation of the
// wave.  Here the stage's own async copies are waited for explicitly (vmcnt)
// before the barrier, LDS reads and writes (lgkmcnt) in the same asm; the
// "memory" clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void rs_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The same copy through a buffer descriptor (32-bit offset from base).  While a
// FLAT copy is outstanding the compiler waits lgkmcnt(0) before every LDS read
// use; with this form it keeps exact waits.
__device__ __forceinline__ void rs_bcopy16(const void* base, uint32_t voff, uint32_t soff, void* lds_wave_base) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds_wave_base, 16, int(voff), int(soff), 0, 0);
}

__device__ __forceinline__ void rs_copy16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// An NVFP4 group scale (e4m3 code) split as s = 2^e * m for the dequantisation
// below: the f32 value s (whose exponent is 2^e) and m = s / 2^e in fp16, at most
// four significant bits, the sign of s included.
struct NvScale {
  float s;
  f16x2 m;
};
__device__ __forceinline__ NvScale nv_scale(uint32_t code) {
  // e4m3 -> fp16 without a branch: the code's exponent and mantissa bits placed
  // as an fp16 pattern read 2^-8 times the value (e4m3 subnormals become fp16
  // subnormals), and 2^8 times that is exact
  const uint32_t hb = ((code & 0x7Fu) << 7) | ((code & 0x80u) << 8);
  const _Float16 h = __builtin_bit_cast(_Float16, uint16_t(hb)) * _Float16(256.0f);
  const uint32_t mh = (uint32_t(__builtin_bit_cast(uint16_t, h)) & 0x83FFu) | 0x3C00u;
  return NvScale{float(h), __builtin_bit_cast(f16x2, mh | (mh << 16))};
}

// Eight e2m1 codes (one dword, low nibble = lower k) times a group scale -> eight
// fp16 values in k order.  The fp4 conversion applies 2^e (it takes only the
// exponent of its f32 scale operand), one packed multiply per pair applies m; the
// e2m1 value times 2^e and then times m are exact in fp16.
__device__ __forceinline__ f16x8 e2m1x8_to_f16(uint32_t w, NvScale sc) {
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.s, 0) * sc.m;
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.s, 1) * sc.m;
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.s, 2) * sc.m;
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc.s, 3) * sc.m;
  return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// Activation ring storage in LDS, one variable per (size, ID) instantiation.
template <int N, int ID>
__device__ __forceinline__ uint8_t* rs_lds_slot() {
  __shared__ __attribute__((aligned(1024))) uint8_t a[N];
  return a;
}

__device__ __forceinline__ i32x8 rs_cat(uint4 lo, uint4 hi) {
  return i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

// Packed fp4 weight-scale layout: for each block of 32 consecutive weight rows and
// each 256 input channels, the 32 rows' 256/G scale bytes (G = 32 for MXFP4, 16 for
// NVFP4) are stored row after row.  Byte offset of scale group kg (channels
// G*kg .. G*kg+G-1) of weight row `row` in a matrix whose rows hold rowlen channels
// (a multiple of 256; the matrix's row count a multiple of 32).
template <int G>
__host__ __device__ __forceinline__ size_t fp4_scale_offset(size_t row, int rowlen, int kg) {
  constexpr int SPR = 256 / G;                     // scale bytes of one row per 256 channels
  return ((row >> 5) * size_t(rowlen / 256) + size_t(kg / SPR)) * (32 * SPR) + (row & 31) * SPR + kg % SPR;
}

// One thread per (weight row, 256 channels): the row's SPR bytes from the row-major
// [rows][rowlen/G] layout into the packed one.  Threads run in packed order so the
// stores are contiguous.
template <int G>
__global__ __launch_bounds__(256) void pack_fp4_scales_kernel(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst, int64_t rows, int rowlen) {
  constexpr int SPR = 256 / G;
  using V = std::conditional_t<SPR == 8, uint2, uint4>;
  const int nst = rowlen / 256;
  const int64_t n = rows * nst;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t blk = i >> 5, r = i & 31, rb = blk / nst;
    const int st = int(blk - rb * nst);
    const int64_t row = rb * 32 + r;
    const V v = *reinterpret_cast<const V*>(src + row * (rowlen / G) + size_t(st) * SPR);
    *reinterpret_cast<V*>(dst + fp4_scale_offset<G>(size_t(row), rowlen, st * SPR)) = v;
  }
}

}  // namespace

// WPE: minimum waves per SIMD the register allocation must leave room for; BUF:
// activation copies through a buffer descriptor (A's extent below 4 GiB).
template <int MS, int MODE, int RECIPE, int NST, int WPE = 1, bool BUF = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) void ffn_rs_kernel(GemmArgs g) {
  constexpr int BM = MS * 32;
  constexpr bool BF16 = RECIPE == MOE_RECIPE_BF16;
  constexpr bool MX = RECIPE == MOE_RECIPE_MXFP4;
  constexpr bool FP8 = RECIPE == MOE_RECIPE_FP8_B128;
  constexpr bool NV = RECIPE == MOE_RECIPE_NVFP4;
  constexpr bool FP4 = MX || NV;                   // packed e2m1 weights with per-row scale bytes
  constexpr bool ASC = FP8 || MX;                  // activations as codes plus row scales
  constexpr int EA = (BF16 || NV) ? 2 : 1;         // activation bytes per element (NVFP4: fp16 values)
  // K per stage: 128 weight bytes of every row, except MXFP4's down GEMM (K =
  // intermediate, a short loop), whose two-stage ring pays one stage's load and
  // one stage's compute per tile without overlap: 128-deep stages halve both
  constexpr int KS = FP4 ? ((MX && MODE == EPI_STORE) ? 128 : 256) : RS_ROWB / EA;
  constexpr int AROWB = KS * EA;                   // activation bytes per LDS row and stage
  constexpr int CPR = AROWB / 16;                  // 16-byte chunks per LDS row
  constexpr int EBW = BF16 ? 2 : 1;                // weight bytes per element (bf16 2, fp8 1; fp4 half)
  constexpr int WROWB = FP4 ? KS / 2 : KS * EBW;   // weight bytes per row and stage
  constexpr int BCH = WROWB / 32;                  // 16-byte weight chunks per lane, fragment and stage
  constexpr int SG = MX ? 32 : 16;                 // fp4 scale group along K
  constexpr int A_INSTR = MS * CPR / 8;            // async copies per wave per stage: BM*CPR chunks / 256 lanes
  // per-row activation scales of a stage (fp8: fp32 bits of one scale; MX: KS/32
  // E8M0 bytes) and a lane's weight scales of a stage (its half: MX KS/64 E8M0
  // bytes; NVFP4 8 e4m3 bytes)
  using SaT = std::conditional_t<MX && KS == 256, uint2, uint32_t>;
  using SbT = std::conditional_t<NV, uint2, std::conditional_t<KS == 256, uint32_t, uint16_t>>;
  static_assert(size_t(NST) * BM * (AROWB + sizeof(SaT)) + 4 * BM * 4 <= 160 * 1024, "LDS budget");
  // fp8: one LDS variable per activation ring slot, so that the compiler knows
  // the copies into the next slot do not write the one being read and does not
  // wait for them before the stage's LDS reads.  (The other recipes keep one
  // ring array: split, they measured no faster, and MXFP4 spilled more.)
  constexpr int SLOT = BM * AROWB;
  static_assert(NST >= 2 && NST <= 3, "two or three ring slots");
  auto As = [&](int b) -> uint8_t* {
    if constexpr (FP8) {
      if constexpr (NST >= 3)
        return b == 0 ? rs_lds_slot<SLOT, 0>() : (b == 1 ? rs_lds_slot<SLOT, 1>() : rs_lds_slot<SLOT, 2>());
      else
        return b == 0 ? rs_lds_slot<SLOT, 0>() : rs_lds_slot<SLOT, 1>();
    } else {
      return rs_lds_slot<NST * SLOT, 3>() + b * SLOT;
    }
  };
  __shared__ SaT Sa[NST][BM];
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
  // this lane's weight bytes for the stage at k0, per fragment: its half of the
  // row's WROWB contiguous bytes
  auto bsrc = [&](int f, int k0) -> const uint8_t* { return brow[f] + koff(k0) + half * (WROWB / 2); };
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
  // fp4 weight scales of fragment f at k0 for this lane's half of the stage: MX
  // E8M0 per 32 (groups k0/32 + (KS/64)h ..), NVFP4 e4m3 per 16 (k0/16 + 8h .. +7),
  // in the packed layout (fp4_scale_offset): a wave's 32 rows read one contiguous
  // run of whole lines per stage.  Per lane a fixed base; the stage adds a
  // wave-uniform offset.
  const uint8_t* sb_base[2];
  if constexpr (FP4) {
    const uint8_t* S = static_cast<const uint8_t*>(g.B_scale);
#pragma unroll
    for (int f = 0; f < 2; ++f)
      sb_base[f] = S + (MODE == EPI_SWIGLU
                            ? fp4_scale_offset<SG>(size_t(sub0) * 2 * ns + ncol[f], K, half * (KS / SG / 2))
                            : fp4_scale_offset<SG>(size_t(ti.e) * g.n_experts_split * g.N + ncol[f], ns,
                                                   half * (KS / SG / 2)));
  }
  auto bscale_fp4 = [&](int f, int k0) -> SbT {
    constexpr int RUN = 32 * 256 / SG;             // bytes of one 32-row block per 256 channels
    size_t off;
    if (MODE == EPI_SWIGLU) off = size_t(k0 / 256) * RUN + (k0 % 256) / SG;
    else off = size_t(k0 / ns) * g.N * (ns / SG) + size_t((k0 % ns) / 256) * RUN + (k0 % 256) / SG;
    return *reinterpret_cast<const SbT*>(sb_base[f] + off);
  };


  // ---- activation copies: copy j of wave w fills LDS chunk positions (w*MS + j)*64 + lane
  std::conditional_t<BUF, uint32_t, const uint8_t*> a_src[A_INSTR];
#pragma unroll
  for (int j = 0; j < A_INSTR; ++j) {
    const int p = (wave * A_INSTR + j) * 64 + lane, r = p / CPR, c = rs_slot<AROWB>(r, p % CPR);
    const size_t off = size_t(a_row(g, ti.row0 + min(r, ti.rows - 1))) * g.lda * EA + c * 16;
    if constexpr (BUF) a_src[j] = uint32_t(off);
    else a_src[j] = A + off;
  }
  const int sa_row = ASC ? a_row(g, ti.row0 + min(tid % BM, ti.rows - 1)) : 0;
  auto load_sa = [&](int k0) -> SaT {            // (rows clamped)
    if constexpr (MX)
      return *reinterpret_cast<const SaT*>(static_cast<const uint8_t*>(g.A_scale) + size_t(sa_row) * (K / 32) + k0 / 32);
    else
      return __float_as_uint(static_cast<const float*>(g.A_scale)[size_t(sa_row) * (K / 128) + k0 / 128]);
  };

  uint4 breg[NST][2][BCH];
  SaT sreg[NST];
  SbT sbm[NST][2];
  float sbf[NST][2];                               // fp8: the stage's two weight-block scales
  auto issue = [&](int k0, int buf) {
#pragma unroll
    for (int j = 0; j < A_INSTR; ++j)
      if constexpr (BUF) rs_bcopy16(A, a_src[j], uint32_t(k0 * EA), As(buf) + (wave * A_INSTR + j) * 1024);
      else rs_copy16(a_src[j] + size_t(k0) * EA, As(buf) + (wave * A_INSTR + j) * 1024);
    // fp8 with a two-stage ring (whose waits are vmcnt(0)): only the threads that
    // stage a row scale load it.  Otherwise every thread loads one, so that counted
    // waits match across waves (MXFP4 measured no faster with fewer loads).
    if (ASC && (!FP8 || NST >= 3 || tid < BM)) sreg[buf] = load_sa(k0);
    // every wave loads (inactive column waves read a clamped, valid row) so that all
    // waves count the same loads per stage
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const uint8_t* p = bsrc(f, k0);
#pragma unroll
      for (int c = 0; c < BCH; ++c) breg[buf][f][c] = *reinterpret_cast<const uint4*>(p + c * 16);
      // the weight scales travel with their stage: a load issued at compute time,
      // behind the next stage's weight loads, would make its wait cover those too
      if (FP4) sbm[buf][f] = bscale_fp4(f, k0);
      if (FP8) sbf[buf][f] = bscale_fp8(f, k0);
    }
  };
  constexpr int PER_STAGE = A_INSTR + (ASC ? 1 : 0) + 2 * BCH + (FP4 || FP8 ? 2 : 0);   // loads per stage per thread

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
  // fp4 rings keep their weight loads in flight across the stage barrier
  // (rs_barrier), and rings of three or more stages, and MXFP4's gate/up ring,
  // issue one stage in every iteration (past the end: the last stage again, an L2
  // hit): each wave then always has NST-1 stages in flight and one wait count that
  // the compiler can track covers every iteration.  Otherwise only real stages
  // are issued (a surplus stage holds up the epilogue, which costs a short K loop
  // most), and bf16 and fp8 take a plain __syncthreads() (measured: as fast or
  // faster for them).
  constexpr bool EVERY = FP4 && (NST >= 3 || (MX && MODE == EPI_SWIGLU));
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    if (EVERY) issue((kb + min(s, KT - 1)) * KS, s);
    else if (s < KT) issue((kb + s) * KS, s);
  }

  for (int kt0 = 0; kt0 < KT; kt0 += NST) {
#pragma unroll
    for (int buf = 0; buf < NST; ++buf) {
      const int kt = kt0 + buf;
      if (kt >= KT) break;
      // stage kt's activation copies must have landed in every wave's LDS slots;
      // the weight registers are waited for by the compiler at their first use
      if (EVERY || (NST >= 3 && kt + 1 < KT)) rs_wait_vmcnt<(NST >= 3 ? (NST - 2) * PER_STAGE : 0)>();
      else rs_wait_vmcnt<0>();
      if (ASC && tid < BM) Sa[buf][tid] = sreg[buf];
      if constexpr (FP4) rs_barrier();
      else __syncthreads();
      const int nb = (buf + NST - 1) % NST;
      if (EVERY) {
        issue((kb + min(kt + NST - 1, KT - 1)) * KS, nb);
        __builtin_amdgcn_sched_barrier(0);         // the next stage's loads go out before this one's compute
      } else if (kt + NST - 1 < KT) {
        issue((kb + kt + NST - 1) * KS, nb);
      }
      // (fp4: a wave without columns computes on its clamped rows and stores
      // nothing, with no branch around the accumulators)
      if (!FP4 && !wave_on) continue;
      const uint8_t* Ab = As(buf);
      if constexpr (BF16) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 b0 = __builtin_bit_cast(bf16x8, breg[buf][0][s]);
          const bf16x8 b1 = __builtin_bit_cast(bf16x8, breg[buf][1][s]);
#pragma unroll
          for (int i = 0; i < MS; ++i) {
            if (i < act_ms) {
              const bf16x8 a =
                  __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Ab + rs_swz<AROWB>(i * 32 + l32, half * 4 + s)));
              acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[i][0], 0, 0, 0);
              acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[i][1], 0, 0, 0);
            }
          }
        }
      } else if constexpr (NV) {
        // fp16 MFMA on exactly dequantised operands: the activations are fp16 values
        // already; the weights' e2m1 codes become fp16 by a byte lookup, times the
        // group's e4m3 scale (every product is exact in fp16).  Step s takes the
        // stage's k = 128h + 8s .. +8 in lane half h on both sides: dword s of the
        // lane's 64 weight bytes, scale byte s/2 of its eight, activation chunk
        // 16h + s of the row.
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          f16x8 bw[2];
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const uint4 q = breg[buf][f][s >> 2];
            const uint32_t w = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
            const uint32_t sw = (s >> 3) ? sbm[buf][f].y : sbm[buf][f].x;
            bw[f] = e2m1x8_to_f16(w, nv_scale((sw >> (8 * ((s >> 1) & 3))) & 0xffu));
          }
#pragma unroll
          for (int i = 0; i < MS; ++i) {
            // (a single row block always holds rows: no branch, so that the
            // accumulators stay in place, measured faster for NVFP4 only)
            if ((MS == 1 && i == 0) || i < act_ms) {
              const f16x8 a = __builtin_bit_cast(
                  f16x8, *reinterpret_cast<const uint4*>(Ab + rs_swz<AROWB>(i * 32 + l32, 16 * half + s)));
              acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bw[0], a, acc[i][0], 0, 0, 0);
              acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bw[1], a, acc[i][1], 0, 0, 0);
            }
          }
        }
      } else if constexpr (FP8) {
        const float sb0 = sbf[buf][0], sb1 = sbf[buf][1];
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          if (i >= act_ms) continue;
          const int ar = i * 32 + l32;
          i32x8 a[2];
#pragma unroll
          for (int s = 0; s < 2; ++s)
            a[s] = rs_cat(*reinterpret_cast<const uint4*>(Ab + rs_swz<AROWB>(ar, 4 * half + 2 * s)),
                          *reinterpret_cast<const uint4*>(Ab + rs_swz<AROWB>(ar, 4 * half + 2 * s + 1)));
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
        // MFMA m of the stage's KS/64: weight lane half h holds the stage's K
        // (KS/2)h + 32m .. +32 (window block h); the fp8 operand lane half h the
        // matching K 32m + 16h .. +16 (chunk 2m + h) and KS/2 + 32m + 16h .. +16
        // (chunk KS/32 + 2m + h); both scales of lane (row, h) are group
        // (KS/64)h + m of the stage.
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          if (i >= act_ms) continue;
          const int ar = i * 32 + l32;
          uint32_t saw;                              // this lane's half of the row's stage scales
          if constexpr (KS == 256) {
            const uint2 sa8 = Sa[buf][ar];
            saw = half ? sa8.y : sa8.x;
          } else {
            saw = Sa[buf][ar] >> (16 * half);
          }
#pragma unroll
          for (int m = 0; m < KS / 64; ++m) {
            const i32x8 a = rs_cat(*reinterpret_cast<const uint4*>(Ab + rs_swz<AROWB>(ar, 2 * m + half)),
                                   *reinterpret_cast<const uint4*>(Ab + rs_swz<AROWB>(ar, KS / 32 + 2 * m + half)));
            const int sa = int((saw >> (8 * m)) & 0xffu);
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const uint4 bw = breg[buf][f][m];
              const i32x8 b = i32x8{int(bw.x), int(bw.y), int(bw.z), int(bw.w), 0, 0, 0, 0};
              acc[i][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  b, a, acc[i][f], 4, 0, 0, int((uint32_t(sbm[buf][f]) >> (8 * m)) & 0xffu), 0, sa);
            }
          }
        }
      }
    }
  }
  // The surplus stages issued past the end (EVERY) may still be copying into LDS:
  // a workgroup must not end with copies into LDS that a later one may own.
  if constexpr (EVERY) rs_wait_vmcnt<0>();

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

template <int MODE, int RECIPE, bool BUF>
static void rs_launch_t(int ms, dim3 grid, const GemmArgs& g, hipStream_t st) {
  if constexpr (RECIPE != MOE_RECIPE_FP8_B128) {
    if (ms >= 4) {                                 // 128-row tiles, held to two waves per SIMD
      ffn_rs_kernel<4, MODE, RECIPE, 2, 2, BUF><<<grid, 256, 0, st>>>(g);
      return;
    }
  }
  if constexpr (RECIPE == MOE_RECIPE_FP8_B128) {
    if (ms == 3) {                                 // 96-row tiles (fp8's 128-row tile spills), two waves per SIMD
      ffn_rs_kernel<3, MODE, RECIPE, 2, 2, BUF><<<grid, 256, 0, st>>>(g);
      return;
    }
  }
  // NVFP4's stages carry fp16 activations four times as deep as bf16's: one more stage in flight
  if (ms <= 1)
    ffn_rs_kernel<1, MODE, RECIPE, (RECIPE == MOE_RECIPE_NVFP4 ? 3 : RS_NST1), 1, BUF><<<grid, 256, 0, st>>>(g);
  else
    ffn_rs_kernel<2, MODE, RECIPE, RS_NST2, (RECIPE == MOE_RECIPE_FP8_B128 ? 2 : 1), BUF><<<grid, 256, 0, st>>>(g);
}

// The fp4 recipes copy activations through buffer descriptors when A's extent
// (a_rows known) is below 4 GiB (measured: MXFP4 gate/up 2.37 -> 2.18 ms; bf16
// decode was slower that way, 3.19 -> 3.66 ms, and keeps the FLAT form).  A
// library built with MOE_FORCE_FLAT_COPIES=1 always takes the FLAT form.
template <int MODE, int RECIPE>
static void rs_launch(int ms, dim3 grid, const GemmArgs& g, hipStream_t st) {
  if constexpr (RECIPE == MOE_RECIPE_MXFP4 || RECIPE == MOE_RECIPE_NVFP4 || RECIPE == MOE_RECIPE_FP8_B128) {
    constexpr int64_t ea = RECIPE == MOE_RECIPE_NVFP4 ? 2 : 1;
    if (!MOE_FORCE_FLAT_COPIES && g.a_rows > 0 && g.a_rows * g.lda * ea < (int64_t(1) << 32) - 256) {
      rs_launch_t<MODE, RECIPE, true>(ms, grid, g, st);
      return;
    }
  }
  rs_launch_t<MODE, RECIPE, false>(ms, grid, g, st);
}

template <int MODE>
static hipError_t rs_launch_recipe(int recipe, int ms, dim3 grid, const GemmArgs& g, hipStream_t st) {
  if (recipe == MOE_RECIPE_BF16) rs_launch<MODE, MOE_RECIPE_BF16>(ms, grid, g, st);
  else if (recipe == MOE_RECIPE_FP8_B128) rs_launch<MODE, MOE_RECIPE_FP8_B128>(ms, grid, g, st);
  else if (recipe == MOE_RECIPE_NVFP4) rs_launch<MODE, MOE_RECIPE_NVFP4>(ms, grid, g, st);
  else rs_launch<MODE, MOE_RECIPE_MXFP4>(ms, grid, g, st);
  return hipGetLastError();
}

// Tiles of ms*32 rows (ms = 1 or 2; bf16, MXFP4 and NVFP4 also 4, fp8 also 3).  bf16 is used for the shared experts of every
// bf16-activation recipe as well.
hipError_t launch_rs_swiglu(int recipe, int ms, int m_tiles, const GemmArgs& g, hipStream_t st) {
  return rs_launch_recipe<EPI_SWIGLU>(recipe, ms, dim3(g.N / 128, m_tiles), g, st);
}
// ksplit > 1: fp32 partial products of ksplit equal K ranges (K / 64 / ksplit stages
// each, an integer), see GemmArgs::split_stride.
hipError_t launch_rs_down(int recipe, int ms, int m_tiles, const GemmArgs& g, hipStream_t st, int ksplit) {
  return rs_launch_recipe<EPI_STORE>(recipe, ms, dim3((g.N + RS_NB - 1) / RS_NB, m_tiles, ksplit), g, st);
}

hipError_t launch_pack_fp4_scales(int recipe, int64_t rows, int rowlen, const void* src, void* dst, hipStream_t st) {
  const int64_t n = rows * (rowlen / 256);
  const int grid = int(std::min<int64_t>((n + 255) / 256, 65536));
  const uint8_t* s = static_cast<const uint8_t*>(src);
  uint8_t* d = static_cast<uint8_t*>(dst);
  if (recipe == MOE_RECIPE_MXFP4) pack_fp4_scales_kernel<32><<<grid, 256, 0, st>>>(s, d, rows, rowlen);
  else pack_fp4_scales_kernel<16><<<grid, 256, 0, st>>>(s, d, rows, rowlen);
  return hipGetLastError();
}

}  // namespace moe
