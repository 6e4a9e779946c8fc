// Internal launchers of the MoE library (host side); every one enqueues on `st`
// and returns hipGetLastError().
#pragma once

#include "common.h"

namespace moe {

// Pairs per block of the counting sort.
constexpr int PERM_CHUNK = 1024;

inline int perm_blocks(int pairs) { return (pairs + PERM_CHUNK - 1) / PERM_CHUNK; }

// Instrumentation (moe_profile_start / moe_profile_stop): while recording, each
// launch is bracketed by two events on its stream.  No-ops otherwise.
void prof_begin(hipStream_t st);
void prof_end(int tag, hipStream_t st);
struct ProfScope {
  int tag;
  hipStream_t st;
  ProfScope(int t, hipStream_t s) : tag(t), st(s) { prof_begin(s); }
  ~ProfScope() { prof_end(tag, st); }
};

// Route scratch (gate logits or screened partial sums, split gate weights, norms).
size_t route_workspace_bytes(const moe_config_t& c);
hipError_t launch_route(const moe_config_t& c, const void* x, const float* gate_w, const float* bias,
                        int32_t* topk_idx, float* topk_w, void* route_ws, hipStream_t st);

hipError_t launch_permute(const moe_config_t& c, const int32_t* topk_idx, const void* x, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, void* x_perm, void* x_perm_scale,
                          int32_t* hist_ws, hipStream_t st);
hipError_t launch_quantize_tokens(const moe_config_t& c, const void* x, void* xq, void* xq_scale, hipStream_t st);

// Scratch of the grouped FFN: tile lists + SwiGLU output h (+ its scales).
struct FfnScratch {
  int32_t* tiles_l;      // tiles of experts with many rows (LDS-staged kernel)
  int32_t* tiles_s;      // tiles of experts with few rows (register-streaming kernel)
  void* h;               // [T*k][I] activation format
  void* h_scale;         // fp32 [T*k][I/128] or E8M0 [T*k][I/32]
};

// Rows per tile of the LDS-staged kernel: bf16 256; fp8 192, whose smaller
// activation slots leave room in LDS for a third weight slot.
constexpr int LDS_ROWS_BF16 = 256;
constexpr int LDS_ROWS_FP8 = 192;

// How the routed experts' rows are cut into tiles and which kernel runs them.
struct FfnPlan {
  bool f32;              // fp32 recipe: VALU kernel, 16-row tiles (list S only)
  int thresh;            // experts with >= thresh rows go to list L
  bool nt;               // list L's weight copies take the non-temporal cache policy
  int bm_l, bm_s;        // rows per tile of each list
  int max_l, max_s;      // grid bounds of each list
  int tile_group;        // list L's tile order (GemmArgs::tile_group)
};
FfnPlan ffn_plan(const moe_config_t& c);

// a_map (nullable): pair row p reads activation row a_map[p] / top_k of x_perm (the
// fused gather: x_perm then holds the token rows in token order).
hipError_t launch_grouped_ffn(const moe_config_t& c, const int32_t* offsets, const void* x_perm,
                              const void* x_perm_scale, const int32_t* a_map, const moe_weights_t& w, void* y_perm,
                              const FfnScratch& s, hipStream_t st);

// resid (nullable): residual rows [T][H] added to the output.
hipError_t launch_combine(const moe_config_t& c, const void* y_perm, const int32_t* pair_pos, const float* topk_w,
                          const void* x, const moe_weights_t* shared, const void* resid, void* out, void* h_shared,
                          float* sh_out, float* sh_part, hipStream_t st);

// MXFP4 / NVFP4 weight scales from the row-major [rows][rowlen/G] layout into the packed
// one the register-streaming kernels read (rows % 32 == 0, rowlen % 256 == 0).
hipError_t launch_pack_fp4_scales(int recipe, int64_t rows, int rowlen, const void* src, void* dst, hipStream_t st);

// MXFP4 weights [rows][row_len] -> e4m3fn codes with fp32 scales per 128 x 128 block
// (rows, row_len multiples of 128); inexact (nullable) counts blocks not reproduced exactly.
hipError_t launch_mxfp4_to_fp8(int64_t rows, int row_len, const void* q, const void* e8, void* out, float* out_scale,
                               int32_t* inexact, hipStream_t st);

hipError_t launch_rmsnorm(const moe_config_t& c, const void* h, const float* w, float eps, void* x, hipStream_t st);

}  // namespace moe
