// Grouped expert GEMMs for prefill-sized expert blocks (moe_infer's per-expert
// gate/up/down + SiLU over contiguous row blocks: DeepSeek-V3 walk-through,
// pwwt.cn/news/5781524, section 3.4), bf16 and fp8 (128x128 block scales).
//
// Tile: up to 32*MS rows x 256 weight rows (SwiGLU: 128 gate_proj rows and the
// matching 128 up_proj rows; down: 256 output columns) on a WM x WN grid of
// wavefronts.  Wave (wm, wn) owns the 32-row fragments wm, wm+WM, wm+2WM, ... and
// 8/WN of the eight 32-wide weight fragments (SwiGLU: 4/WN gate fragments and the
// matching up fragments, so that SiLU(g)*u pairs sit in the same lane and
// register).  A partial tile (the last rows of an expert) skips the same share of
// row fragments in every wave and costs MFMA time in proportion to its rows.
//
// Both operands are staged through LDS with gfx950's direct global->LDS 16-byte
// loads into rings of 128-byte rows (64 bf16 or 128 fp8 of K per stage; whole
// cache lines per row): two activation slots and three weight slots, so that the
// weight copies run two stages ahead (tiles of 256 rows for bf16, 192 for fp8,
// whose scale slots leave no room for the third weight slot at 256 rows).  The copies
// use the buffer-descriptor form (buffer_load_dwordx4 ... lds, 32-bit offsets)
// when the tensors allow it: while a FLAT-form copy (global_load_lds_dwordx4) is
// outstanding, the compiler cannot order the LDS fragment reads against it and
// waits for all of them before every MFMA group.
//
// The 16-byte chunk c of LDS row r sits at slot
// c ^ ((r ^ (r>>1)) & 7): any 16 consecutive rows reading one chunk hit 16
// distinct 16-byte slots of a 256-byte bank window.  The XOR is applied on the
// global side, so the LDS writes of one copy instruction (64 lanes x 16 bytes)
// stay contiguous as the hardware requires.
//
// bf16 runs v_mfma_f32_32x32x16_bf16 in 16-deep sub-steps whose operands are read
// from LDS while the previous sub-step's MFMAs run.  fp8 runs
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales, one per 16x16 block and
// stage, so that a block's stage sum needs no dependent MFMA chain; the 128x128
// block scales are applied with one FMA per accumulator element and stage
// (stage sum x row scale x weight scale, both staged through LDS with the
// operands).
//
// Tiles are numbered (row tile, column tile) and mapped so that consecutive
// numbers run on the same XCD: column tile fastest, so that the column tiles
// sharing an activation block meet in that XCD's L2; or, when experts span many
// row tiles, in groups of 8 row tiles with row tile fastest (GemmArgs::
// tile_group), so that the row tiles of a heavy expert also share its weight
// blocks.  With the first order the row tiles of one expert read the same weight
// rows far apart in time, so each of them streams the weights from HBM again;
// experts of 257..511 rows pay two weight passes.
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int ROWB = 128;        // bytes of K per LDS row and stage
constexpr int NST = 2;           // stages in the LDS ring

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Slot of logical 16-byte chunk c in LDS row r.
__device__ __forceinline__ int swz_slot(int r, int c) { return c ^ ((r ^ (r >> 1)) & 7); }

// Async global -> LDS copy through a buffer descriptor (MUBUF): unlike the FLAT
// form, an outstanding copy of this kind does not stop the compiler from
// counting LDS reads (lgkmcnt) precisely.
// CPOL: cache policy bits of the copy (0, or CPOL_NT: non-temporal).
constexpr int CPOL_NT = 2;
template <int CPOL = 0>
__device__ __forceinline__ void buf_copy16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds_wave_base, 16, int(voff), int(soff), 0, CPOL);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), -1, 0x00020000);
}

template <int CPOL = 0>
__device__ __forceinline__ void async_copy16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_wave_base, 16, 0, CPOL);
}

// s_waitcnt with vmcnt = n, other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

enum Kind { KIND_BF16 = 0, KIND_FP8 = 1 };

__device__ __forceinline__ i32x8 cat(uint4 lo, uint4 hi) {
  return i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ float max_over_lanes16(float v) {   // within each 16-lane group
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace

// Row offset of weight fragment f within a wave's share of the tile's NB weight
// rows: SwiGLU (SPLIT = gate fragments per wave) takes its gate fragments from
// rows 0..NB/2-1 and the matching up fragments from rows NB/2..NB-1.
template <int SPLIT, int NB>
__device__ constexpr int bfrag_row(int f) { return SPLIT > 0 ? (f < SPLIT ? 0 : NB / 2) + (f % SPLIT) * 32 : f * 32; }

// fp8 scale staging (separate LDS variables, instantiated by the fp8 kernels only)
template <int N, int ID>
__device__ __forceinline__ float* lds_f32() {
  __shared__ __attribute__((aligned(16))) float a[N];
  return a;
}

// A third weight slot (instantiated by the PIPE 2 kernels only)
template <int N>
__device__ __forceinline__ uint8_t* lds_wslot2() {
  __shared__ __attribute__((aligned(1024))) uint8_t a[N];
  return a;
}

// Workgroup barrier that leaves vector memory loads in flight: __syncthreads()
// releases every address space and waits for all of them (vmcnt(0)); here each
// wave has already waited, by count, for the copies the next stage needs.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One fp8 stage (128 K, one 128-block of both scale grids) for the NU 16-row
// blocks of this wave that hold real rows.  Row block u: rows
// (wm + WM*(u>>1))*32 + 16*(u&1) + 0..15; column block c = 2f + cb: weight
// fragment f, columns 16*cb + 0..15.  Operand lane l: row / column l & 15, K bytes
// 32*(l>>4) .. +32 of the stage (the same K order on both sides).  The weight
// block is the MFMA's first operand, so accumulator lane l, register r holds
// column 4*(l>>4) + r of token row l & 15: one row scale per lane and row block.
// Sp: the stage's row scales, MU per lane in row-block order (see the kernel's
// scale staging); sbv: its two weight scales; sbi[f]: which one fragment f takes.
template <int NU, int MU, int NC, int WM, int SPLIT, int NB>
__device__ __forceinline__ void stage_fp8(f32x4 (&acc)[MU][NC], const uint8_t* As_buf, const uint8_t* Bw,
                                          const float* Sp, const float (&sbv)[2], const int (&sbi)[NC / 2], int wm,
                                          int r16, int kg) {
  const int lo0 = r16 * ROWB + (swz_slot(r16, 2 * kg) << 4);     // rows read are 16*m + r16
  const int lo1 = r16 * ROWB + (swz_slot(r16, 2 * kg + 1) << 4);
  i32x8 bv[NC], av[2];
  f32x4 part[NC];
  float sa[MU];
#pragma unroll
  for (int q = 0; q < MU / 2; ++q) {            // (MU * 4 bytes per lane: 8-byte aligned)
    const float2 v = *reinterpret_cast<const float2*>(Sp + (wm * 16 + r16) * MU + 2 * q);
    sa[2 * q] = v.x; sa[2 * q + 1] = v.y;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint8_t* p = Bw + (bfrag_row<SPLIT, NB>(c >> 1) + 16 * (c & 1)) * ROWB;
    bv[c] = cat(lds16(p + lo0), lds16(p + lo1));
  }
  auto rd = [&](int u, int slot) {
    const int row = (wm + WM * (u >> 1)) * 32 + 16 * (u & 1);
    const uint8_t* p = As_buf + row * ROWB;
    av[slot] = cat(lds16(p + lo0), lds16(p + lo1));
  };
  auto fma_blk = [&](int u) {
    const float rs[2] = {sa[u] * sbv[0], sa[u] * sbv[1]};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u][c][r] = fmaf(part[c][r], rs[sbi[c >> 1]], acc[u][c][r]);
  };
  rd(0, 0);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    // The unit's NC MFMAs back to back, then the next unit's LDS reads, then this
    // unit's scale FMAs: each FMA reads an MFMA result that the later MFMAs' issue
    // time has already covered, and the FMAs cover the LDS reads' latency.
#pragma unroll
    for (int c = 0; c < NC; ++c)
      part[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv[c], av[u & 1], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0,
                                                                 127, 0, 127);
    sched_fence();
    if (u + 1 < NU) rd(u + 1, (u + 1) & 1);
    sched_fence();
    fma_blk(u);
    sched_fence();
  }
}

// MS: 32-row fragments per tile; WM x WN: wavefront grid; PIPE: the main loop,
// both with two activation slots and three weight slots, so that each stage's
// weight copies have two stages of compute to land -- 2 (bf16): the stage
// barrier sits before the stage's last sub-step, so that stage k+2's copies and
// stage k+1's first LDS reads overlap stage k's last MFMAs; 3 (fp8): the barrier
// at the stage start, the scales staged with the activations; NB: weight rows
// per tile (SwiGLU: NB/2 h columns).  NTB: the weight copies take the
// non-temporal cache policy, for launches in which each expert's weights are
// read by one row tile only (nothing later reuses them from L2 or the MALL):
// full-line non-temporal reads streamed at 7.1 TB/s on the box against 6.3 for
// the default policy, and took a bf16 decode layer step from 4.89 to 4.39 ms.
template <int MS, int MODE, int KIND, int WM, int WN, int PIPE, int NB, bool BUF, bool NTB = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void ffn_lds_kernel(GemmArgs g) {
  constexpr int NW = WM * WN;                       // wavefronts
  constexpr int BM = MS * 32;
  constexpr int MW = MS / WM;                       // row fragments per wave
  constexpr int NF = NB / 32 / WN;                  // weight fragments per wave
  constexpr int NFG = NF / 2;                       // SwiGLU: gate (= up) fragments per wave
  constexpr int SPLIT = (MODE == EPI_SWIGLU) ? NFG : 0;
  constexpr int A_INSTR = BM * (ROWB / 16) / 64 / NW;   // async copies per wave per stage (A)
  constexpr int B_INSTR = NB * (ROWB / 16) / 64 / NW;   // (B)
  static_assert(MW >= 1 && NFG >= 1 && A_INSTR >= 1 && B_INSTR >= 1, "tile shape");
  static_assert(BM * (ROWB / 16) == A_INSTR * 64 * NW && NB * (ROWB / 16) == B_INSTR * 64 * NW, "copy cover");
  constexpr bool FP8 = KIND == KIND_FP8;
  static_assert(!FP8 || NB == 256, "fp8 re-quantisation needs the tile's 128 h columns");
  constexpr int EB = FP8 ? 1 : 2;                   // bytes per element
  constexpr int KS = ROWB / EB;                     // K per stage
  // One LDS variable per ring slot and role: the compiler then knows that the
  // copies into one slot and the reads of the other do not overlap, and issues no
  // wait for the copies in flight before the reads.
  static_assert(NST == 2, "two ring slots");
  __shared__ __attribute__((aligned(1024))) uint8_t As0[BM * ROWB], As1[BM * ROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs0[NB * ROWB], Bs1[NB * ROWB];
  float *Sa0 = nullptr, *Sa1 = nullptr, *Sb0 = nullptr, *Sb1 = nullptr, *amax_lds = nullptr;
  if constexpr (FP8) {
    Sa0 = lds_f32<BM, 0>();                          // row scales
    Sa1 = lds_f32<BM, 1>();
    Sb0 = lds_f32<4, 2>();                           // weight scales
    Sb1 = lds_f32<4, 3>();
    amax_lds = lds_f32<WN * BM, 4>();                // epilogue
  }

  const int ncols = (MODE == EPI_SWIGLU) ? g.N / (NB / 2) : (g.N + NB - 1) / NB;
  const int V = ncols * row_tiles(g, BM);
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  if (b >= V) return;
  const int tnum = xcd_tile(b, V);
  // g.tile_group > 1 (launches whose experts span several row tiles): the ~32
  // workgroups an XCD holds at once cover tile_group row tiles x a few column
  // tiles and share weight and activation blocks in L2; otherwise column tile
  // fastest, so that the column tiles of a row tile share its activations.
  int mt, nt;
  tile_coords(tnum, V, ncols, g.tile_group, mt, nt);
  TileInfo ti;
  tile_info(g, BM, mt, ti);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int K = g.K, ns = g.nsplit;
  const uint8_t* A = static_cast<const uint8_t*>(g.A);
  const uint8_t* B = static_cast<const uint8_t*>(g.B);
  const int act_ms = (ti.rows + 31) >> 5;           // 32-row fragments holding real rows

  // ---- global sources of this thread's async copies: copy j of wave w fills LDS
  // chunk positions p = (w*INSTR + j)*64 + lane -> row p / 8, slot p % 8, logical
  // chunk slot ^ key(row)
  // (BUF: byte offsets below 2^32 from A and from the tile's expert weights, copied
  // through buffer descriptors; else 64-bit addresses, copied with the FLAT form)
  using Src = std::conditional_t<BUF, uint32_t, const uint8_t*>;
  Src a_src[A_INSTR];
#pragma unroll
  for (int j = 0; j < A_INSTR; ++j) {
    const int p = (wave * A_INSTR + j) * 64 + lane, r = p / (ROWB / 16);
    const int c = swz_slot(r, p % (ROWB / 16));
    const size_t off = size_t(a_row(g, ti.row0 + min(r, ti.rows - 1))) * g.lda * EB + c * 16;
    if constexpr (BUF) a_src[j] = uint32_t(off);
    else a_src[j] = A + off;
  }
  int n0, sub0 = 0;
  if (MODE == EPI_SWIGLU) {
    n0 = nt * (NB / 2);
    sub0 = ti.e * g.n_experts_split + n0 / ns;
  } else {
    n0 = nt * NB;
  }
  const uint8_t* const B0 = B + (MODE == EPI_SWIGLU ? size_t(sub0) * 2 * ns * size_t(K)
                                                    : size_t(ti.e) * g.n_experts_split * g.N * ns) * EB;
  Src b_src[B_INSTR];
#pragma unroll
  for (int j = 0; j < B_INSTR; ++j) {
    const int p = (wave * B_INSTR + j) * 64 + lane, r = p / (ROWB / 16);
    const int c = swz_slot(r, p % (ROWB / 16));
    size_t rowoff;
    if (MODE == EPI_SWIGLU) {
      const int wr = (r < NB / 2) ? (n0 % ns + r) : (ns + n0 % ns + r - NB / 2);
      rowoff = size_t(wr) * size_t(K);
    } else {
      const int n = min(n0 + r, g.N - 1);
      rowoff = size_t(n) * ns;
    }
    if constexpr (BUF) b_src[j] = uint32_t(rowoff * EB + c * 16);
    else b_src[j] = B0 + rowoff * EB + c * 16;
  }
  auto copy_a = [&](int j, int k0, void* lds) {
    if constexpr (BUF) buf_copy16(buf_rsrc(A), a_src[j], uint32_t(k0 * EB), lds);
    else async_copy16(a_src[j] + size_t(k0) * EB, lds);
  };
  auto copy_b = [&](int j, size_t ko, void* lds) {
    if constexpr (BUF) buf_copy16<NTB ? CPOL_NT : 0>(buf_rsrc(B0), b_src[j], uint32_t(ko), lds);
    else async_copy16<NTB ? CPOL_NT : 0>(b_src[j] + ko, lds);
  };
  auto koff_bytes = [&](int k0) -> size_t {
    if (MODE == EPI_SWIGLU) return size_t(k0) * EB;
    return (size_t(k0 / ns) * g.N * ns + (k0 % ns)) * EB;
  };
  // fp8 scales of the stage at k0, loaded only by the threads that stage them in
  // LDS (the fp8 loop waits for all of a wave's loads, vmcnt(0), so the waves need
  // not count the same loads): sa = activation scale of tile row tid (tid < BM,
  // rows clamped); sb = weight scale q = tid (tid < 2; SwiGLU: q = 0 gate block,
  // 1 up block; down: q = 128-column block of the tile's 256 columns).  Each sa
  // load is a 4-byte read from its own token row; with half of them (and the
  // register-streaming kernel's likewise) a skewed fp8 layer step took 1.6% less.
  float sa_reg[NST], sb_reg[NST];
  const int sa_row = FP8 ? a_row(g, ti.row0 + min(tid % BM, ti.rows - 1)) : 0;   // this thread's A-scale row
  // LDS position of tile row tid's scale: lane r16 of the waves with row offset wm
  // finds its MW*2 row blocks' scales at (wm*16 + r16)*2*MW + u
  int sa_pos = 0;
  if constexpr (FP8) {
    const int r = tid % BM, i = r >> 5;
    sa_pos = ((i % WM) * 16 + (r & 15)) * (2 * MW) + 2 * (i / WM) + ((r >> 4) & 1);
  }
  auto load_scales = [&](int k0, int buf) {
    if (FP8 && tid < BM) {
      const float* SA = static_cast<const float*>(g.A_scale);
      sa_reg[buf] = SA[size_t(sa_row) * (K / 128) + k0 / 128];
    }
    if (FP8 && tid < 2) {
      const float* SB = static_cast<const float*>(g.B_scale);
      const int q = tid;
      if (MODE == EPI_SWIGLU) {
        const int rb = (q * ns + n0 % ns) / 128;
        sb_reg[buf] = SB[(size_t(sub0) * (2 * ns / 128) + rb) * (K / 128) + k0 / 128];
      } else {
        const int sub = ti.e * g.n_experts_split + k0 / ns;
        const int cb = min(n0 + q * 128, g.N - 1) / 128;
        sb_reg[buf] = SB[(size_t(sub) * (g.N / 128) + cb) * (ns / 128) + (k0 % ns) / 128];
      }
    }
  };
  // Tile-relative weight column of each of this wave's fragments (SwiGLU: the h
  // column block of the gate/up pair); the wave's first LDS weight row.
  int fcol[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) fcol[f] = (MODE == EPI_SWIGLU) ? (wn * NFG + f % NFG) * 32 : (wn * NF + f) * 32;
  const int brow0 = (MODE == EPI_SWIGLU) ? wn * NFG * 32 : wn * NF * 32;
  // row fragments of this wave that hold real rows (wave-uniform)
  const int nj = min(MW, max(0, (act_ms - wm + WM - 1) / WM));

  // accumulators: bf16 32x32 fragments [MW][NF]; fp8 16x16 blocks [2*MW][2*NF]
  f32x16 acc16[FP8 ? 1 : MW][FP8 ? 1 : NF];
  f32x4 acc4[FP8 ? 2 * MW : 1][FP8 ? 2 * NF : 1];
  if constexpr (FP8) {
#pragma unroll
    for (int u = 0; u < 2 * MW; ++u)
#pragma unroll
      for (int c = 0; c < 2 * NF; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc4[u][c][r] = 0.0f;
  } else {
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc16[i][f][r] = 0.0f;
  }
  int sbi[NF];                                      // fp8: weight-scale index of fragment f
#pragma unroll
  for (int f = 0; f < NF; ++f) sbi[f] = (MODE == EPI_SWIGLU) ? (f < NFG ? 0 : 1) : fcol[f] / 128;

  const int KT = K / KS;
  if constexpr (PIPE == 2 && !FP8) {
    // ---- bf16 main loop, activation ring of 2 slots, weight ring of 3: stage kt
    // reads A slot kt % 2 and B slot kt % 3.  At the barrier of stage kt, stage
    // kt+1 must have landed while stage kt+2's weights (issued last) may still be
    // in flight; then stage kt+2's activations and stage kt+3's weights refill the
    // slots stage kt has finished reading.
    constexpr int NS = ROWB / 32;
    const int half = lane >> 5, l32 = lane & 31;
    uint8_t* const Bs2 = lds_wslot2<NB * ROWB>();
    auto Asl = [&](auto ac) -> uint8_t* { return decltype(ac)::value == 0 ? As0 : As1; };
    auto Bsl = [&](auto bc) -> uint8_t* {
      return decltype(bc)::value == 0 ? Bs0 : (decltype(bc)::value == 1 ? Bs1 : Bs2);
    };
    auto issue_a = [&](int k0, auto ac) {
#pragma unroll
      for (int j = 0; j < A_INSTR; ++j)
        if ((wave * A_INSTR + j) * (1024 / ROWB) < ti.rows)
          copy_a(j, k0, Asl(ac) + (wave * A_INSTR + j) * 1024);
    };
    auto issue_b = [&](int k0, auto bc) {          // B_INSTR copies per wave, always
      const size_t ko = koff_bytes(k0);
#pragma unroll
      for (int j = 0; j < B_INSTR; ++j) copy_b(j, ko, Bsl(bc) + (wave * B_INSTR + j) * 1024);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    auto mainloop = [&](auto njc) {
      constexpr int NJ = decltype(njc)::value;
      constexpr int NJA = NJ > 0 ? NJ : 1;
      bf16x8 bv[2][NF], av[2][NJA];
      auto rd = [&](auto ac, auto bc, int s, int slot) {
        if constexpr (NJ > 0) {
          const int off = l32 * ROWB + (swz_slot(l32, 2 * s + half) << 4);
          const uint8_t* Aw = Asl(ac) + wm * 32 * ROWB + off;
          const uint8_t* Bw = Bsl(bc) + brow0 * ROWB + off;
#pragma unroll
          for (int f = 0; f < NF; ++f) bv[slot][f] = __builtin_bit_cast(bf16x8, lds16(Bw + bfrag_row<SPLIT, NB>(f) * ROWB));
#pragma unroll
          for (int j = 0; j < NJ; ++j) av[slot][j] = __builtin_bit_cast(bf16x8, lds16(Aw + WM * 32 * ROWB * j));
        }
      };
      auto mm = [&](int slot) {
        if constexpr (NJ > 0) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int f = 0; f < NF; ++f)
              acc16[j][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[slot][f], av[slot][j], acc16[j][f], 0, 0, 0);
        }
      };
      auto step = [&](int kt, auto ac, auto bc) {
        constexpr int a = decltype(ac)::value, b = decltype(bc)::value;
#pragma unroll
        for (int s = 0; s < NS - 1; ++s) {
          rd(ac, bc, s + 1, (s + 1) & 1);
          sched_fence();
          mm(s & 1);
          sched_fence();
        }
        if (kt + 1 < KT) {
          if (kt + 2 < KT) wait_vmcnt<B_INSTR>();   // stage kt+1 has landed (own copies)
          else wait_vmcnt<0>();
          lds_barrier();                              // (everyone's); everyone is done reading stage kt
          if (kt + 2 < KT) issue_a((kt + 2) * KS, ac);
          if (kt + 3 < KT) issue_b((kt + 3) * KS, bc);
        }
        rd(std::integral_constant<int, a ^ 1>{}, std::integral_constant<int, (b + 1) % 3>{}, 0, 0);
        sched_fence();
        mm((NS - 1) & 1);
        sched_fence();
      };
      rd(I0{}, I0{}, 0, 0);
      int kt = 0;
      for (; kt + 5 < KT; kt += 6) {
        step(kt, I0{}, I0{});
        step(kt + 1, I1{}, I1{});
        step(kt + 2, I0{}, I2{});
        step(kt + 3, I1{}, I0{});
        step(kt + 4, I0{}, I1{});
        step(kt + 5, I1{}, I2{});
      }
      if (kt < KT) step(kt, I0{}, I0{});
      if (kt + 1 < KT) step(kt + 1, I1{}, I1{});
      if (kt + 2 < KT) step(kt + 2, I0{}, I2{});
      if (kt + 3 < KT) step(kt + 3, I1{}, I0{});
      if (kt + 4 < KT) step(kt + 4, I0{}, I1{});
    };
    issue_a(0, I0{});
    issue_b(0, I0{});
    if (KT > 1) {
      issue_a(KS, I1{});
      issue_b(KS, I1{});
    }
    if (KT > 2) issue_b(2 * KS, I2{});
    wait_vmcnt<0>();                                // (a wave's copy count varies with the tile's rows)
    __syncthreads();
    if (MW >= 4 && nj == 4) mainloop(std::integral_constant<int, (MW >= 4 ? 4 : 0)>{});
    else if (MW >= 3 && nj == 3) mainloop(std::integral_constant<int, (MW >= 3 ? 3 : 0)>{});
    else if (MW >= 2 && nj == 2) mainloop(std::integral_constant<int, (MW >= 2 ? 2 : 0)>{});
    else if (nj == 1) mainloop(std::integral_constant<int, 1>{});
    else mainloop(std::integral_constant<int, 0>{});
  } else if constexpr (PIPE == 3 && FP8) {
    // ---- fp8 main loop, activation (and scale) ring of 2 slots, weight ring of 3:
    // stage kt reads A / scale slot kt % 2 and B slot kt % 3.  At the top of stage
    // kt a wave waits, by count, for its own copies of stage kt while stage kt+1's
    // weights (issued last) stay in flight; after the barrier it refills the slots
    // stage kt-1 has finished with: stage kt+1's activations and scales, then stage
    // kt+2's weights.  The weight copies thus have two stages of compute to land.
    uint8_t* const Bs2 = lds_wslot2<NB * ROWB>();
    auto Asl = [&](auto ac) -> uint8_t* { return decltype(ac)::value == 0 ? As0 : As1; };
    auto Bsl = [&](auto bc) -> uint8_t* {
      return decltype(bc)::value == 0 ? Bs0 : (decltype(bc)::value == 1 ? Bs1 : Bs2);
    };
    // Activation copies, then the stage's scales.  Unlike the other loops, every
    // copy is issued, also those of rows past the tile's last real row (they read
    // that row again): with the copies under a branch, the compiler no longer
    // tells their LDS slot from the one being read and makes each stage wait for
    // the next stage's activations before its first LDS read.
    auto issue_a = [&](int k0, auto ac) {
      constexpr int a = decltype(ac)::value;
#pragma unroll
      for (int j = 0; j < A_INSTR; ++j) copy_a(j, k0, Asl(ac) + (wave * A_INSTR + j) * 1024);
      load_scales(k0, a);
    };
    auto issue_b = [&](int k0, auto bc) {          // B_INSTR copies per wave, always
      const size_t ko = koff_bytes(k0);
#pragma unroll
      for (int j = 0; j < B_INSTR; ++j) copy_b(j, ko, Bsl(bc) + (wave * B_INSTR + j) * 1024);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    const int r16 = lane & 15, kg = lane >> 4;
    constexpr int MU = 2 * MW, NC = 2 * NF;
    // FULL: the steady state, where stages kt+1 and kt+2 exist and the copies are
    // issued without a branch.  (With a branch around them, the compiler's own
    // wait before the scale writes can no longer count the weight copies that
    // follow the scale loads on every path, and it waits for all of them.)
    auto step = [&](auto fullc, int kt, auto ac, auto bc) {
      constexpr bool FULL = decltype(fullc)::value;
      constexpr int a = decltype(ac)::value, b = decltype(bc)::value;
      if (FULL || kt + 1 < KT) wait_vmcnt<B_INSTR>();   // all but stage kt+1's weights
      else wait_vmcnt<0>();
      float* const sa_l = a == 0 ? Sa0 : Sa1;
      float* const sb_l = a == 0 ? Sb0 : Sb1;
      if (tid < BM) sa_l[sa_pos] = sa_reg[a];
      if (tid < 2) sb_l[tid] = sb_reg[a];
      lds_barrier();                                // everyone's stage kt landed; stage kt-1 read
      // (scheduling barriers keep the issue order: the scale loads must precede
      // the weight copies that the next stage's wait leaves in flight)
      sched_fence();
      if (FULL || kt + 1 < KT) issue_a((kt + 1) * KS, std::integral_constant<int, a ^ 1>{});
      sched_fence();
      if (FULL || kt + 2 < KT) issue_b((kt + 2) * KS, std::integral_constant<int, (b + 2) % 3>{});
      sched_fence();
      const float sbv[2] = {sb_l[0], sb_l[1]};
      const uint8_t* Ab = Asl(ac);
      const uint8_t* Bw = Bsl(bc) + brow0 * ROWB;
      // (the row-fragment count is dispatched here, inside the step: one loop per
      // count made the compiler move the units' MFMAs together and spill)
      if (MW >= 4 && nj == 4) stage_fp8<(MW >= 4 ? 8 : 2), MU, NC, WM, SPLIT, NB>(acc4, Ab, Bw, sa_l, sbv, sbi, wm, r16, kg);
      else if (MW >= 3 && nj == 3) stage_fp8<(MW >= 3 ? 6 : 2), MU, NC, WM, SPLIT, NB>(acc4, Ab, Bw, sa_l, sbv, sbi, wm, r16, kg);
      else if (MW >= 2 && nj == 2) stage_fp8<(MW >= 2 ? 4 : 2), MU, NC, WM, SPLIT, NB>(acc4, Ab, Bw, sa_l, sbv, sbi, wm, r16, kg);
      else if (nj == 1) stage_fp8<2, MU, NC, WM, SPLIT, NB>(acc4, Ab, Bw, sa_l, sbv, sbi, wm, r16, kg);
    };
    using F = std::true_type;
    using T = std::false_type;
    issue_a(0, I0{});
    sched_fence();
    issue_b(0, I0{});
    if (KT == 1) {
      sched_fence();
      step(T{}, 0, I0{}, I0{});
    } else {
      // (stage 1's weights issued on every path into the loop, so that the
      // compiler's count of the copies in flight is the same on all of them)
      issue_b(KS, I1{});
      sched_fence();
      int kt = 0;
      for (; kt + 7 < KT; kt += 6) {
        step(F{}, kt, I0{}, I0{});
        step(F{}, kt + 1, I1{}, I1{});
        step(F{}, kt + 2, I0{}, I2{});
        step(F{}, kt + 3, I1{}, I0{});
        step(F{}, kt + 4, I0{}, I1{});
        step(F{}, kt + 5, I1{}, I2{});
      }
      step(T{}, kt, I0{}, I0{});                      // the last 2..7 stages
      step(T{}, kt + 1, I1{}, I1{});
      if (kt + 2 < KT) step(T{}, kt + 2, I0{}, I2{});
      if (kt + 3 < KT) step(T{}, kt + 3, I1{}, I0{});
      if (kt + 4 < KT) step(T{}, kt + 4, I0{}, I1{});
      if (kt + 5 < KT) step(T{}, kt + 5, I1{}, I2{});
      if (kt + 6 < KT) step(T{}, kt + 6, I0{}, I0{});
    }
  } else {
    static_assert(PIPE == 2 || PIPE == 3, "bf16 runs the PIPE 2 loop, fp8 the PIPE 3 loop");
  }

  // ---- epilogues
  if constexpr (!FP8) {
    // 32x32 accumulator layout, weight fragment as the MFMA's first operand: lane
    // l, register r = 4q + e holds token row l & 31 and column 8q + 4*(l>>5) + e of
    // the fragment, so each lane stores runs of four consecutive columns
    const int l32 = lane & 31, c4 = 4 * (lane >> 5);
    auto pack4 = [](float a, float b, float c, float d) {
      return uint2{uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16),
                   uint32_t(f32_to_bf16(c)) | (uint32_t(f32_to_bf16(d)) << 16)};
    };
    if (MODE == EPI_SWIGLU) {
      uint16_t* Hh = static_cast<uint16_t*>(g.out);
#pragma unroll
      for (int j = 0; j < MW; ++j) {
        const int i = wm + WM * j;
        const int row = i * 32 + l32;
        if (i >= act_ms || row >= ti.rows) continue;
        uint16_t* hrow = Hh + size_t(ti.row0 + row) * g.ldo + n0;
#pragma unroll
        for (int f = 0; f < NFG; ++f) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = swiglu_f32(acc16[j][f][4 * q + e], acc16[j][f + NFG][4 * q + e], g.swiglu_limit);
            *reinterpret_cast<uint2*>(hrow + fcol[f] + 8 * q + c4) = pack4(h[0], h[1], h[2], h[3]);
          }
        }
      }
    } else {  // EPI_STORE: bf16 y rows, or fp32 rows (out_f32)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (n0 + fcol[f] >= g.N) continue;            // partial column tile (g.N % 128 == 0)
#pragma unroll
        for (int j = 0; j < MW; ++j) {
          const int i = wm + WM * j;
          const int row = i * 32 + l32;
          if (i >= act_ms || row >= ti.rows) continue;
          const size_t o = size_t(ti.row0 + row) * g.ldo + n0 + fcol[f] + c4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc16[j][f];
            if (g.out_f32)
              *reinterpret_cast<float4*>(static_cast<float*>(g.out) + o + 8 * q) =
                  float4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
            else
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + o + 8 * q) =
                  pack4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
        }
      }
    }
  } else {
    // 16x16 accumulator layout: block (u, c) lane l register r -> tile row
    // (wm + WM*(u>>1))*32 + 16*(u&1) + (l&15), column fcol[c>>1] + 16*(c&1) + 4*(l>>4) + r
    constexpr int NC = 2 * NF;
    const int r16 = lane & 15, kg = lane >> 4;
    if (MODE == EPI_SWIGLU) {
      // h re-quantised per (row, 128 columns): the tile's 128 h columns are one
      // block, split over the WN column waves and, within a wave, over the four
      // lanes of a row
      uint8_t* Hq = static_cast<uint8_t*>(g.out);
#pragma unroll
      for (int u = 0; u < 2 * MW; ++u) {
        const int row = (wm + WM * (u >> 1)) * 32 + 16 * (u & 1) + r16;
        const bool on = (wm + WM * (u >> 1)) < act_ms;
        float hv[NC / 2][4];
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < NC / 2; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            hv[c][r] = swiglu_f32(acc4[u][c][r], acc4[u][c + NC / 2][r], g.swiglu_limit);
            m = fmaxf(m, fabsf(hv[c][r]));
          }
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (on && kg == 0) amax_lds[wn * BM + row] = m;
        __syncthreads();
        if (on && row < ti.rows) {
          float amax = amax_lds[row];
#pragma unroll
          for (int q = 1; q < WN; ++q) amax = fmaxf(amax, amax_lds[q * BM + row]);
          const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
          uint8_t* hrow = Hq + size_t(ti.row0 + row) * g.ldo + n0;
#pragma unroll
          for (int c = 0; c < NC / 2; ++c) {
            uint32_t packed = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) packed |= uint32_t(f32_to_e4m3(hv[c][r] / sc)) << (8 * r);
            *reinterpret_cast<uint32_t*>(hrow + fcol[c >> 1] + 16 * (c & 1) + 4 * kg) = packed;
          }
          if (wn == 0 && kg == 0) static_cast<float*>(g.out_scale)[size_t(ti.row0 + row) * (g.N / 128) + n0 / 128] = sc;
        }
        __syncthreads();
      }
    } else {  // EPI_STORE: four consecutive columns per lane
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (n0 + fcol[c >> 1] >= g.N) continue;       // partial column tile (g.N % 128 == 0)
        const int col = n0 + fcol[c >> 1] + 16 * (c & 1) + 4 * kg;
#pragma unroll
        for (int u = 0; u < 2 * MW; ++u) {
          if ((wm + WM * (u >> 1)) >= act_ms) continue;
          const int row = (wm + WM * (u >> 1)) * 32 + 16 * (u & 1) + r16;
          if (row >= ti.rows) continue;
          const size_t o = size_t(ti.row0 + row) * g.ldo + col;
          if (g.out_f32) {
            *reinterpret_cast<float4*>(static_cast<float*>(g.out) + o) =
                float4{acc4[u][c][0], acc4[u][c][1], acc4[u][c][2], acc4[u][c][3]};
          } else {
            const uint32_t lo = uint32_t(f32_to_bf16(acc4[u][c][0])) | (uint32_t(f32_to_bf16(acc4[u][c][1])) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16(acc4[u][c][2])) | (uint32_t(f32_to_bf16(acc4[u][c][3])) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + o) = uint2{lo, hi};
          }
        }
      }
    }
  }
}

template <int MS, int MODE, int KIND, bool BUF, int WM, int WN, int PIPE = 0, int NB = 256, bool NTB = false>
void launch_lds_variant(const GemmArgs& g, int m_tiles, hipStream_t st) {
  constexpr size_t lds = size_t(NST) * (MS * 32 + NB) * ROWB + (PIPE >= 2 ? size_t(NB) * ROWB : 0) +
                         (KIND == KIND_FP8 ? size_t(NST + WN) * MS * 32 * 4 + 32 : 0);
  static_assert(lds <= 160 * 1024, "LDS budget");
  const int ncols = (MODE == EPI_SWIGLU) ? g.N / (NB / 2) : (g.N + NB - 1) / NB;
  ffn_lds_kernel<MS, MODE, KIND, WM, WN, PIPE, NB, BUF, NTB><<<dim3(ncols, m_tiles), 64 * WM * WN, 0, st>>>(g);
}

// Production configurations: 256-row tiles on 2 x 4 wavefronts (two per SIMD).
// bf16: the stage barrier before the last sub-step and a three-slot weight ring
// (all 160 KB of LDS).  fp8: the block-scale FMAs keep the accumulators in ordinary
// VGPRs, and a second wave per SIMD overlaps one wave's FMAs with the other's MFMAs.
// nt (bf16): non-temporal weight copies (see ffn_lds_kernel's NTB).
template <int MODE, int KIND, bool BUF>
static hipError_t launch_lds_tiles(int m_tiles, const GemmArgs& g, bool nt, hipStream_t st) {
  if constexpr (KIND == KIND_FP8) launch_lds_variant<LDS_ROWS_FP8 / 32, MODE, KIND, BUF, 2, 4, 3>(g, m_tiles, st);
  else if (nt) launch_lds_variant<LDS_ROWS_BF16 / 32, MODE, KIND, BUF, 2, 4, 2, 256, true>(g, m_tiles, st);
  else launch_lds_variant<LDS_ROWS_BF16 / 32, MODE, KIND, BUF, 2, 4, 2>(g, m_tiles, st);
  return hipGetLastError();
}

// Buffer-descriptor copies address A and the tile's expert weights with 32-bit
// offsets: usable when a_rows is known and both extents stay below 4 GiB.  A
// library built with MOE_FORCE_FLAT_COPIES=1 always takes the 64-bit FLAT-copy form
// (the test build exercises it; no shape of the test workloads reaches it otherwise).
template <int MODE, int KIND>
static hipError_t launch_lds_any(int m_tiles, const GemmArgs& g, bool nt, hipStream_t st) {
  constexpr int64_t eb = KIND == KIND_FP8 ? 1 : 2, lim = (int64_t(1) << 32) - 256;
  const int64_t a_bytes = g.a_rows * g.lda * eb;
  const int64_t b_bytes = MODE == EPI_SWIGLU ? 2 * int64_t(g.nsplit) * g.K * eb
                                             : int64_t(g.n_experts_split) * g.N * g.nsplit * eb;
  if (!MOE_FORCE_FLAT_COPIES && g.a_rows > 0 && a_bytes < lim && b_bytes < lim)
    return launch_lds_tiles<MODE, KIND, true>(m_tiles, g, nt, st);
  return launch_lds_tiles<MODE, KIND, false>(m_tiles, g, nt, st);
}

// 256-row tiles (see launch_lds_tiles).
hipError_t launch_lds_swiglu(bool fp8, bool nt, int m_tiles, const GemmArgs& g, hipStream_t st) {
  return fp8 ? launch_lds_any<EPI_SWIGLU, KIND_FP8>(m_tiles, g, false, st)
             : launch_lds_any<EPI_SWIGLU, KIND_BF16>(m_tiles, g, nt, st);
}
hipError_t launch_lds_down(bool fp8, bool nt, int m_tiles, const GemmArgs& g, hipStream_t st) {
  return fp8 ? launch_lds_any<EPI_STORE, KIND_FP8>(m_tiles, g, false, st)
             : launch_lds_any<EPI_STORE, KIND_BF16>(m_tiles, g, nt, st);
}

}  // namespace moe
