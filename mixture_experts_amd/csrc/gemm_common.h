// Tile scheduling shared by the grouped-GEMM kernels.
#pragma once

#include "common.h"

namespace moe {

enum EpiMode { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_COMBINE = 2 };

// Arguments of one grouped (or dense) GEMM launch.
//   Grouped mode (tiles != nullptr): tile i covers rows offsets[e] + m0 .. of expert e,
//   where tiles = {count, e_0, m0_0, e_1, m0_1, ...}.  Dense mode: one expert, rows 0..dense_rows.
struct GemmArgs {
  const void* A;            // activations [rows][K] (bf16, fp32 or fp8 codes)
  int64_t a_rows;           // rows of A a launch may address (0: unknown); lets the
                            // LDS-staged kernel use 32-bit buffer offsets when small
  const void* A_scale;      // activation scales (fp8: fp32 [rows][K/128]; MX: E8M0 [rows][K/32])
  int lda;
  const int32_t* offsets;   // [E+1]
  const int32_t* tiles;
  int dense_rows;
  const void* B;            // weights of expert 0 (see the SwiGLU / down layouts below)
  const void* B_scale;
  int K;                    // reduction length
  int N;                    // output columns (h columns for SwiGLU, hidden for down)
  int nsplit;               // per-sub-expert width: SwiGLU columns (I or Is), down K-split (I or Is)
  int n_experts_split;      // number of sub-experts stacked in one launch (shared experts), else 1
  void* out;                // [rows][N]
  void* out_scale;          // h scales for the quantised recipes
  int ldo;
  int out_f32;              // down projection: store fp32 instead of bf16
  float swiglu_limit;       // SwiGLU epilogue: > 0 clamps gate and up first (swiglu_f32)
  // Fused gather: when a_map is set, the A row (and A-scale row) of pair row p is
  // a_map[p] / a_div -- the token of the p-th sorted (token, slot) pair -- so the
  // GEMM reads the token rows directly instead of a gathered copy.
  const int32_t* a_map;
  int a_div;
  // K split (register-streaming kernel, plain store mode): blockIdx.z takes the
  // z-th of gridDim.z equal K ranges and writes its fp32 partial products to
  // out + z * split_stride.
  size_t split_stride;
  // combine epilogue
  const void* resid;        // residual rows added to the output (nullable)
  const void* y_perm;
  const int32_t* pair_pos;
  const float* topk_w;
  int topk;
  // LDS-staged kernel: > 1 numbers its tiles in groups of tile_group row tiles,
  // row tile fastest within a group (see ffn_lds_kernel); else column tile fastest
  int tile_group;
};

struct TileInfo {
  int e, row0, rows;
};

// Row tile `tile` of a launch: an (expert, first row) entry of the tile list, or a
// BM-row slice of a dense operand.  False when the tile holds no rows.
__device__ __forceinline__ bool tile_info(const GemmArgs& g, int BM, int tile, TileInfo& ti) {
  if (g.tiles) {
    if (tile >= g.tiles[0]) return false;
    ti.e = g.tiles[1 + 2 * tile];
    const int m0 = g.tiles[2 + 2 * tile];
    ti.row0 = g.offsets[ti.e] + m0;
    ti.rows = min(BM, g.offsets[ti.e + 1] - ti.row0);
  } else {
    ti.e = 0;
    ti.row0 = tile * BM;
    ti.rows = min(BM, g.dense_rows - ti.row0);
  }
  return ti.rows > 0;
}

__device__ __forceinline__ bool get_tile(const GemmArgs& g, int BM, TileInfo& ti) {
  return tile_info(g, BM, blockIdx.y, ti);
}

// Row tiles of a launch that holds them (the tile list's count, or the dense slices).
__device__ __forceinline__ int row_tiles(const GemmArgs& g, int BM) {
  return g.tiles ? g.tiles[0] : (g.dense_rows + BM - 1) / BM;
}

// Bijective map of a linear block index b < V to a tile number so that the blocks
// one XCD runs (b % 8 fixed: workgroups are dealt round-robin over the eight XCDs)
// cover a contiguous range of tile numbers and share that XCD's L2.
__host__ __device__ __forceinline__ int xcd_tile(int b, int V) {
  const int q = V >> 3, r = V & 7, x = b & 7, l = b >> 3;
  return (x < r) ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
}

// (row tile mt, column tile nt) of tile number tnum < V = row tiles x ncols.
// group > 1: the numbers come in groups of `group` row tiles x all ncols column
// tiles, row tile fastest within a group (the last group may hold fewer row
// tiles); else column tile fastest.  A bijection either way.
__host__ __device__ __forceinline__ void tile_coords(int tnum, int V, int ncols, int group, int& mt, int& nt) {
  if (group > 1) {
    const int nrt = V / ncols, gr0 = tnum / (group * ncols) * group;
    const int gsz = (group < nrt - gr0) ? group : nrt - gr0, idx = tnum - gr0 * ncols;
    mt = gr0 + idx % gsz;
    nt = idx / gsz;
  } else {
    mt = tnum / ncols;
    nt = tnum - mt * ncols;
  }
}

// A-operand row of pair row p (see GemmArgs::a_map).
__device__ __forceinline__ int a_row(const GemmArgs& g, int p) { return g.a_map ? g.a_map[p] / g.a_div : p; }

// 32x32 MFMA accumulator layout: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace moe
