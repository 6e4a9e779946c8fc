// C ABI of the MoE-layer forward library: argument checks, workspace carving and
// the launch sequence of each entry point (declared and documented in include/moe.h).
#include <algorithm>
#include <climits>
#include <vector>

#include "gemm_common.h"
#include "kernels.h"

namespace moe {

hipError_t launch_rs_swiglu(int recipe, int ms, int m_tiles, const GemmArgs& g, hipStream_t st);
hipError_t launch_rs_down(int recipe, int ms, int m_tiles, const GemmArgs& g, hipStream_t st, int ksplit);
hipError_t launch_f32(int mode, int m_tiles, const GemmArgs& g, hipStream_t st);
hipError_t launch_combine_rows(const moe_config_t& c, const void* y_perm, const int32_t* pair_pos,
                               const float* topk_w, const float* sh, int nsh, const void* resid, void* out,
                               hipStream_t st);
hipError_t launch_swiglu_slabs(const float* part, int nz, int T, int nes, int Is, float limit, uint16_t* h,
                               hipStream_t st);
hipError_t launch_build_tiles2(const int32_t* offsets, int E, int thresh, int bm_large, int bm_small,
                               int32_t* tiles_l, int32_t* tiles_s, hipStream_t st);
// 256-row tiles; nt: non-temporal weight copies (bf16), for weights read by one row tile
hipError_t launch_lds_swiglu(bool fp8, bool nt, int m_tiles, const GemmArgs& g, hipStream_t st);
hipError_t launch_lds_down(bool fp8, bool nt, int m_tiles, const GemmArgs& g, hipStream_t st);

namespace {

bool valid_config(const moe_config_t* c) {
  if (!c) return false;
  if (c->num_tokens < 0 || c->hidden <= 0 || c->intermediate <= 0 || c->num_experts <= 0) return false;
  if (c->num_experts > 1024 || c->top_k < 1 || c->top_k > 16 || c->top_k > c->num_experts) return false;
  if (c->num_shared < 0 || (c->num_shared > 0 && c->shared_intermediate <= 0)) return false;
  if (c->n_group < 1 || c->n_group > 64 || c->num_experts % c->n_group != 0) return false;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return false;
  if (c->n_group > 1 && c->num_experts / c->n_group < 2) return false;
  if (int64_t(c->topk_group) * (c->num_experts / c->n_group) < c->top_k) return false;
  if (c->score_func != MOE_SCORE_SIGMOID && c->score_func != MOE_SCORE_SQRTSOFTPLUS) return false;
  if (c->recipe < MOE_RECIPE_F32 || c->recipe > MOE_RECIPE_NVFP4) return false;
  if (!(c->routed_scaling_factor == c->routed_scaling_factor)) return false;
  if (int64_t(c->num_tokens) * c->top_k > (int64_t(1) << 30)) return false;
  if (!(c->swiglu_limit >= 0.0f && c->swiglu_limit <= 3.0e38f)) return false;   // finite, >= 0
  return true;
}

bool supported_shape(const moe_config_t* c) {
  const int q = (c->recipe == MOE_RECIPE_F32) ? 32 : 128;
  // the fp4 routed GEMMs take 256 K per stage (one 128-byte line of every weight row)
  const bool fp4 = c->recipe == MOE_RECIPE_MXFP4 || c->recipe == MOE_RECIPE_NVFP4;
  const int qr = fp4 ? 256 : q;
  if (c->hidden % qr || c->intermediate % qr) return false;
  if (c->num_shared > 0 && c->shared_intermediate % q) return false;
  return true;
}

size_t act_bytes(const moe_config_t& c) { return c.recipe == MOE_RECIPE_F32 ? 4 : 2; }     // x, y, out
size_t routed_act_bytes(const moe_config_t& c) {                                             // x_perm, h
  // NVFP4 rows are kept as their fp16 values
  return c.recipe == MOE_RECIPE_F32 ? 4 : ((c.recipe == MOE_RECIPE_BF16 || c.recipe == MOE_RECIPE_NVFP4) ? 2 : 1);
}
size_t act_scale_bytes(const moe_config_t& c, int64_t rows, int64_t cols) {
  if (c.recipe == MOE_RECIPE_FP8_B128) return size_t(rows * (cols / 128) * 4);
  if (c.recipe == MOE_RECIPE_MXFP4) return size_t(rows * (cols / 32));
  return 0;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Routed experts with quantised weights and activations.
bool quantised(const moe_config_t& c) {
  return c.recipe == MOE_RECIPE_FP8_B128 || c.recipe == MOE_RECIPE_MXFP4 || c.recipe == MOE_RECIPE_NVFP4;
}
// Quantised activations stored as codes plus a separate scale array (x_perm_scale).
bool act_scaled(const moe_config_t& c) { return c.recipe == MOE_RECIPE_FP8_B128 || c.recipe == MOE_RECIPE_MXFP4; }

int shared_ms(int T) { return T > 32 ? 2 : 1; }   // register-streaming tiles for small token counts

// Shared expert at small token counts (decode): its two GEMMs have too few output
// tiles to fill the chip, so each runs as ks equal K ranges writing fp32 partial
// products (summed in order by the SwiGLU and the combine kernels).
struct SharedSplit {
  bool on;
  int ms, mt, ks1, ks2;   // row-tile size (x32), row tiles, K splits of gate/up and of down
};
SharedSplit shared_split(const moe_config_t& c) {
  SharedSplit s{};
  const int T = c.num_tokens, SI = c.num_shared * c.shared_intermediate;
  if (c.recipe == MOE_RECIPE_F32 || SI == 0 || T == 0 || T > 256) return s;
  s.on = true;
  s.ms = shared_ms(T);
  s.mt = (T + 32 * s.ms - 1) / (32 * s.ms);
  // largest split (<= 16) with whole 64-deep stages, >= 4 stages each, <= 1024 blocks
  auto pick = [&](int ncols, int stages) {
    int best = 1;
    for (int d = 1; d <= 16; ++d)
      if (stages % d == 0 && stages / d >= 4 && int64_t(ncols) * s.mt * d <= 1024) best = d;
    return best;
  };
  s.ks1 = pick(2 * SI / 256, c.hidden / 64);
  s.ks2 = pick((c.hidden + 255) / 256, SI / 64);
  return s;
}

// Scratch layout; the same for every entry point so one size serves all of them.
struct Layout {
  size_t route, hist, tiles_l, tiles_s, h, h_scale, h_shared, sh_out, sh_part, idx, w, offsets, sorted,
      pos, xq, xq_scale, y_perm, xn, total;
};

Layout layout(const moe_config_t& c) {
  Layout L{};
  const int64_t T = c.num_tokens, E = c.num_experts, H = c.hidden, I = c.intermediate, P = T * c.top_k;
  const int64_t SI = int64_t(c.num_shared) * c.shared_intermediate;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(std::max<size_t>(bytes, 1)); return at; };
  L.route = take(route_workspace_bytes(c));
  L.hist = take(size_t(int64_t(perm_blocks(int(P))) * E * 4));
  const FfnPlan fp = ffn_plan(c);
  L.tiles_l = take(size_t((2 * int64_t(fp.max_l) + 1) * 4));
  L.tiles_s = take(size_t((2 * int64_t(fp.max_s) + 1) * 4));
  L.h = take(size_t(P * I) * routed_act_bytes(c));
  L.h_scale = take(act_scale_bytes(c, P, I));
  L.h_shared = take(size_t(T * SI) * act_bytes(c));
  L.sh_out = take(c.recipe == MOE_RECIPE_F32 || SI == 0 ? 0 : size_t(T * H * 4));   // fp32 shared-expert rows
  const SharedSplit ss = shared_split(c);
  L.sh_part = take(ss.on ? size_t(std::max<int64_t>(ss.ks1 * T * 2 * SI, ss.ks2 * T * H)) * 4 : 0);
  L.idx = take(size_t(P * 4));
  L.w = take(size_t(P * 4));
  L.offsets = take(size_t((E + 1) * 4));
  L.sorted = take(size_t(P * 4));
  L.pos = take(size_t(P * 4));
  // moe_forward's once-per-token quantised copy of x for the quantised recipes (the
  // routed GEMMs gather its rows; moe_permute writes the caller's x_perm instead)
  L.xq = take(quantised(c) ? size_t(T * H) * routed_act_bytes(c) : 0);
  L.xq_scale = take(act_scale_bytes(c, T, H));
  L.y_perm = take(size_t(P * H) * act_bytes(c));
  L.xn = take(size_t(T * H) * act_bytes(c));          // normalised rows (moe_forward_residual)
  L.total = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

moe_status_t check_common(const moe_config_t* c, void* ws, size_t ws_bytes) {
  if (!valid_config(c)) return MOE_ERR_INVALID_ARGUMENT;
  if (!supported_shape(c)) return MOE_ERR_UNSUPPORTED;
  if (c->num_tokens == 0) return MOE_OK;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < layout(*c).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}


bool weights_ok(const moe_config_t& c, const moe_weights_t* w) {
  if (!w || !w->w13 || !w->w2) return false;
  if (quantised(c) && (!w->w13_scale || !w->w2_scale)) return false;
  return true;
}

moe_status_t to_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

}  // namespace

// Experts with at least 128 rows run on the LDS-staged kernel (256-row tiles);
// experts with fewer rows, fp8's decode-sized experts and the fp4 recipes run on
// the register-streaming kernel with 32-, 64-, 96- (fp8) or 128-row (bf16, fp4)
// tiles.  bf16 at decode-like loads sends every expert to the LDS-staged kernel
// with non-temporal weight copies (see below).
FfnPlan ffn_plan(const moe_config_t& c) {
  FfnPlan p{};
  const int64_t P = int64_t(c.num_tokens) * c.top_k, E = c.num_experts;
  if (c.recipe == MOE_RECIPE_F32) {
    p.f32 = true;
    p.thresh = INT32_MAX;
    p.bm_l = p.bm_s = 16;
    p.max_l = 0;
    p.max_s = int((P + 15) / 16 + E);
    return p;
  }
  const int64_t avg = P / std::max<int64_t>(1, E);
  p.bm_s = avg <= 40 ? 32 : 64;
  // Size the register-streaming tiles so that a typical expert takes one tile and
  // its weights stream from HBM once: MXFP4 and NVFP4 have no large-tile list; bf16 sends only
  // experts under 128 rows there.  (fp8's 128-row variant spills registers; its
  // 96-row one does not: skewed_fp8 12.19 -> 12.02 ms per step against 64 rows.)
  const bool fp4w = c.recipe == MOE_RECIPE_MXFP4 || c.recipe == MOE_RECIPE_NVFP4;
  if (fp4w) p.bm_s = avg <= 24 ? 32 : avg <= 48 ? 64 : 128;
  else if (c.recipe == MOE_RECIPE_BF16 && avg > 48) p.bm_s = 128;
  else if (c.recipe == MOE_RECIPE_FP8_B128 && avg > 48) p.bm_s = 96;
  // bf16 at decode-like loads (experts average at most 48 rows, so nearly every
  // expert is one row tile): every expert goes to the LDS-staged kernel, whose
  // whole-line weight copies can take the non-temporal policy (each expert's
  // weights are read once); measured 4.93 -> 4.39 ms per bf16 decode step.
  p.nt = c.recipe == MOE_RECIPE_BF16 && avg <= 48;
  p.thresh = fp4w ? INT32_MAX : (p.nt ? 1 : 128);
  p.bm_l = c.recipe == MOE_RECIPE_FP8_B128 ? LDS_ROWS_FP8 : LDS_ROWS_BF16;
  p.max_l = (p.thresh == INT32_MAX || P < p.thresh) ? 0 : int((P + p.bm_l - 1) / p.bm_l + std::min<int64_t>(E, P / p.thresh));
  // Experts averaging more rows than one large tile (a skewed load's heavy experts
  // span many row tiles): list L runs in groups of 8 row tiles, so that an XCD's
  // workgroups share those experts' weights in L2 (skewed_fp8 layer step
  // 10.42 -> 10.18 ms); with experts of one or two row tiles the column-fastest
  // order, which shares each row tile's activations, is faster (bf16 prefill
  // gate/up 4.78 against 5.32 ms grouped).
  p.tile_group = avg > p.bm_l ? 8 : 0;
  const int64_t small_bound = (p.thresh == INT32_MAX) ? (P + p.bm_s - 1) / p.bm_s + E
                                                      : E * ((p.thresh + p.bm_s - 1) / p.bm_s);
  p.max_s = int(std::min<int64_t>((P + p.bm_s - 1) / p.bm_s + E, small_bound));
  return p;
}

hipError_t launch_grouped_ffn(const moe_config_t& c, const int32_t* offsets, const void* x_perm,
                              const void* x_perm_scale, const int32_t* a_map, const moe_weights_t& w, void* y_perm,
                              const FfnScratch& s, hipStream_t st) {
  const FfnPlan fp = ffn_plan(c);
  hipError_t e;
  {
    ProfScope p(MOE_K_TILES, st);
    e = launch_build_tiles2(offsets, c.num_experts, fp.thresh, fp.bm_l, fp.bm_s, s.tiles_l, s.tiles_s, st);
  }
  if (e != hipSuccess) return e;
  const bool fp8 = c.recipe == MOE_RECIPE_FP8_B128;
  GemmArgs g{};
  g.swiglu_limit = c.swiglu_limit;
  g.A = x_perm;
  g.A_scale = x_perm_scale;
  g.a_map = a_map;
  g.a_div = c.top_k;
  g.a_rows = a_map ? int64_t(c.num_tokens) : int64_t(c.num_tokens) * c.top_k;
  g.lda = c.hidden;
  g.offsets = offsets;
  g.B = w.w13;
  g.B_scale = w.w13_scale;
  g.K = c.hidden;
  g.N = c.intermediate;
  g.nsplit = c.intermediate;
  g.n_experts_split = 1;
  g.out = s.h;
  g.out_scale = s.h_scale;
  g.ldo = c.intermediate;
  {
    ProfScope p(MOE_K_FFN_GATE_UP, st);
    if (fp.f32) {
      g.tiles = s.tiles_s;
      e = launch_f32(EPI_SWIGLU, fp.max_s, g, st);
    } else {
      if (fp.max_l > 0) {
        g.tiles = s.tiles_l;
        g.tile_group = fp.tile_group;
        e = launch_lds_swiglu(fp8, fp.nt, fp.max_l, g, st);
        g.tile_group = 0;
      }
      if (e == hipSuccess) {
        g.tiles = s.tiles_s;
        e = launch_rs_swiglu(c.recipe, fp.bm_s / 32, fp.max_s, g, st);
      }
    }
  }
  if (e != hipSuccess) return e;
  GemmArgs d = g;
  d.A = s.h;
  d.A_scale = s.h_scale;
  d.a_map = nullptr;                                   // h rows are in pair order
  d.a_rows = int64_t(c.num_tokens) * c.top_k;
  d.lda = c.intermediate;
  d.B = w.w2;
  d.B_scale = w.w2_scale;
  d.K = c.intermediate;
  d.N = c.hidden;
  d.nsplit = c.intermediate;
  d.out = y_perm;
  d.out_scale = nullptr;
  d.ldo = c.hidden;
  ProfScope p(MOE_K_FFN_DOWN, st);
  if (fp.f32) {
    d.tiles = s.tiles_s;
    return launch_f32(EPI_STORE, fp.max_s, d, st);
  }
  if (fp.max_l > 0) {
    d.tiles = s.tiles_l;
    d.tile_group = fp.tile_group;
    e = launch_lds_down(fp8, fp.nt, fp.max_l, d, st);
    d.tile_group = 0;
    if (e != hipSuccess) return e;
  }
  d.tiles = s.tiles_s;
  return launch_rs_down(c.recipe, fp.bm_s / 32, fp.max_s, d, st, 1);
}

hipError_t launch_combine(const moe_config_t& c, const void* y_perm, const int32_t* pair_pos, const float* topk_w,
                          const void* x, const moe_weights_t* shared, const void* resid, void* out, void* h_shared,
                          float* sh_out, float* sh_part, hipStream_t st) {
  if (c.num_shared == 0) {
    ProfScope p(MOE_K_COMBINE, st);
    return launch_combine_rows(c, y_perm, pair_pos, topk_w, nullptr, 0, resid, out, st);
  }
  const int T = c.num_tokens, SI = c.num_shared * c.shared_intermediate;
  hipError_t e;
  const SharedSplit ss = shared_split(c);
  if (ss.on) {
    // gate/up rows of all shared experts as one [2*SI][H] matrix, K split
    GemmArgs g{};
    g.A = x;
    g.lda = c.hidden;
    g.dense_rows = T;
    g.B = shared->w13;
    g.K = c.hidden;
    g.N = 2 * SI;
    g.nsplit = c.hidden;
    g.n_experts_split = 1;
    g.out = sh_part;
    g.ldo = 2 * SI;
    g.out_f32 = 1;
    g.split_stride = size_t(T) * 2 * SI;
    {
      ProfScope p(MOE_K_SHARED_GATE_UP, st);
      e = launch_rs_down(MOE_RECIPE_BF16, ss.ms, ss.mt, g, st, ss.ks1);
      if (e == hipSuccess)
        e = launch_swiglu_slabs(sh_part, ss.ks1, T, c.num_shared, c.shared_intermediate, c.swiglu_limit,
                                static_cast<uint16_t*>(h_shared), st);
    }
    if (e != hipSuccess) return e;
    GemmArgs d{};
    d.A = h_shared;
    d.lda = SI;
    d.dense_rows = T;
    d.B = shared->w2;
    d.K = SI;
    d.N = c.hidden;
    d.nsplit = c.shared_intermediate;
    d.n_experts_split = c.num_shared;
    d.out = sh_part;
    d.ldo = c.hidden;
    d.out_f32 = 1;
    d.split_stride = size_t(T) * c.hidden;
    {
      ProfScope p(MOE_K_SHARED_DOWN_COMBINE, st);
      e = launch_rs_down(MOE_RECIPE_BF16, ss.ms, ss.mt, d, st, ss.ks2);
    }
    if (e != hipSuccess) return e;
    ProfScope p(MOE_K_COMBINE, st);
    return launch_combine_rows(c, y_perm, pair_pos, topk_w, sh_part, ss.ks2, resid, out, st);
  }
  // Prefill-sized token counts (T > 256; fewer take the K split above): the
  // LDS-staged kernel's 256-row tiles, or the fp32 kernel.
  const bool f32 = c.recipe == MOE_RECIPE_F32;
  const int BM = f32 ? 16 : 256, mt = (T + BM - 1) / BM;
  GemmArgs g{};
  g.swiglu_limit = c.swiglu_limit;
  g.A = x;
  g.a_rows = T;
  g.lda = c.hidden;
  g.dense_rows = T;
  g.B = shared->w13;
  g.K = c.hidden;
  g.N = SI;
  g.nsplit = c.shared_intermediate;
  g.n_experts_split = c.num_shared;
  g.out = h_shared;
  g.ldo = SI;
  {
    ProfScope p(MOE_K_SHARED_GATE_UP, st);
    e = f32 ? launch_f32(EPI_SWIGLU, mt, g, st) : launch_lds_swiglu(false, false, mt, g, st);
  }
  if (e != hipSuccess) return e;
  GemmArgs d = g;
  d.A = h_shared;
  d.lda = SI;
  d.B = shared->w2;
  d.K = SI;
  d.N = c.hidden;
  d.ldo = c.hidden;
  if (f32) {                                           // fp32: put-back sum fused into the down projection
    d.out = out;
    d.resid = resid;
    d.y_perm = y_perm;
    d.pair_pos = pair_pos;
    d.topk_w = topk_w;
    d.topk = c.top_k;
    ProfScope p(MOE_K_SHARED_DOWN_COMBINE, st);
    return launch_f32(EPI_COMBINE, mt, d, st);
  }
  d.out = sh_out;                                      // fp32 shared rows, summed with the routed rows next
  d.out_f32 = 1;
  {
    ProfScope p(MOE_K_SHARED_DOWN_COMBINE, st);
    e = launch_lds_down(false, false, mt, d, st);
  }
  if (e != hipSuccess) return e;
  ProfScope p(MOE_K_COMBINE, st);
  return launch_combine_rows(c, y_perm, pair_pos, topk_w, sh_out, 1, resid, out, st);
}

// ---------------------------------------------------------------- instrumentation
namespace {
struct ProfState {
  bool on = false;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;   // 2 per launch
  std::vector<int> tag;
};
ProfState g_prof;
}  // namespace

void prof_begin(hipStream_t st) {
  if (g_prof.on && g_prof.n < g_prof.cap) (void)hipEventRecord(g_prof.ev[2 * g_prof.n], st);
}
void prof_end(int tag, hipStream_t st) {
  if (g_prof.on && g_prof.n < g_prof.cap) {
    (void)hipEventRecord(g_prof.ev[2 * g_prof.n + 1], st);
    g_prof.tag[g_prof.n++] = tag;
  }
}

}  // namespace moe

using namespace moe;

// DeepseekV3MoE.forward on activation rows x, plus (resid != nullptr) the
// residual rows added in the combine.
static hipError_t forward_impl(const moe_config_t& c, const void* x, const void* resid, const float* gate_w,
                               const float* bias, const moe_weights_t* experts, const moe_weights_t* shared,
                               void* out, int32_t* topk_idx_out, float* topk_w_out, void* ws, hipStream_t st) {
  const Layout L = layout(c);
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.idx);
  float* w = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* pos = at<int32_t>(ws, L.pos);
  void* xq = at<void>(ws, L.xq);
  void* xq_scale = act_scaled(c) ? at<void>(ws, L.xq_scale) : nullptr;
  void* y_perm = at<void>(ws, L.y_perm);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  hipError_t e = launch_route(c, x, gate_w, bias, idx, w, at<void>(ws, L.route), st);
  // Fused gather: the routed GEMMs read the token rows of x (or of its quantised
  // copy, made once per token) through the sorted pair order, with no gathered copy.
  if (e == hipSuccess) e = launch_permute(c, idx, x, offsets, sorted, pos, nullptr, nullptr, at<int32_t>(ws, L.hist), st);
  if (e == hipSuccess && quantised(c)) e = launch_quantize_tokens(c, x, xq, xq_scale, st);
  if (e == hipSuccess) {
    FfnScratch sc{at<int32_t>(ws, L.tiles_l), at<int32_t>(ws, L.tiles_s), at<void>(ws, L.h), at<void>(ws, L.h_scale)};
    e = launch_grouped_ffn(c, offsets, quantised(c) ? xq : x, xq_scale, sorted, *experts, y_perm, sc, st);
  }
  if (e == hipSuccess)
    e = launch_combine(c, y_perm, pos, w, x, shared, resid, out, at<void>(ws, L.h_shared), at<float>(ws, L.sh_out),
                       at<float>(ws, L.sh_part), st);
  return e;
}

extern "C" {

size_t moe_workspace_bytes(const moe_config_t* cfg) {
  if (!valid_config(cfg) || !supported_shape(cfg)) return 0;
  return layout(*cfg).total;
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or recipe";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

moe_status_t moe_profile_start(int32_t max_launches) {
  if (max_launches <= 0 || g_prof.on) return MOE_ERR_INVALID_ARGUMENT;
  g_prof.ev.assign(2 * size_t(max_launches), nullptr);
  g_prof.tag.assign(size_t(max_launches), 0);
  for (auto& e : g_prof.ev)
    if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_LAUNCH;
  g_prof.cap = max_launches;
  g_prof.n = 0;
  g_prof.on = true;
  return MOE_OK;
}

moe_status_t moe_profile_stop(double* ms_out, int64_t* count_out, int32_t n_tags) {
  if (!g_prof.on) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = MOE_OK;
  for (int t = 0; t < n_tags; ++t) {
    if (ms_out) ms_out[t] = 0.0;
    if (count_out) count_out[t] = 0;
  }
  for (int i = 0; i < g_prof.n; ++i) {
    float ms = 0.0f;
    if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) {
      st = MOE_ERR_LAUNCH;
      continue;
    }
    const int t = g_prof.tag[i];
    if (t < n_tags) {
      if (ms_out) ms_out[t] += ms;
      if (count_out) count_out[t] += 1;
    }
  }
  for (auto e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof = ProfState{};
  return st;
}

const char* moe_kernel_tag_name(int32_t tag) {
  static const char* names[MOE_K_COUNT] = {"gate_logits", "router", "perm_hist", "perm_scan", "perm_scatter",
                                           "gather", "tile_list", "ffn_gate_up", "ffn_down", "shared_gate_up",
                                           "shared_down_combine", "combine", "rmsnorm"};
  return (tag >= 0 && tag < MOE_K_COUNT) ? names[tag] : "unknown";
}

moe_status_t moe_route(const moe_config_t* cfg, const void* x, const float* gate_w, const float* bias,
                       int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t s = check_common(cfg, ws, ws_bytes);
  if (s != MOE_OK || cfg->num_tokens == 0) return s;
  if (!x || !gate_w || !bias || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = layout(*cfg);
  return to_status(launch_route(*cfg, x, gate_w, bias, topk_idx, topk_w, at<void>(ws, L.route),
                                static_cast<hipStream_t>(stream)));
}

moe_status_t moe_permute(const moe_config_t* cfg, const int32_t* topk_idx, const void* x, int32_t* expert_offsets,
                         int32_t* sorted_pair, int32_t* pair_pos, void* x_perm, void* x_perm_scale, void* ws,
                         size_t ws_bytes, void* stream) {
  moe_status_t s = check_common(cfg, ws, ws_bytes);
  if (s != MOE_OK || cfg->num_tokens == 0) return s;
  if (!topk_idx || !x || !expert_offsets || !sorted_pair || !pair_pos || !x_perm) return MOE_ERR_INVALID_ARGUMENT;
  if (act_scaled(*cfg) && !x_perm_scale) return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = layout(*cfg);
  return to_status(launch_permute(*cfg, topk_idx, x, expert_offsets, sorted_pair, pair_pos, x_perm, x_perm_scale,
                                  at<int32_t>(ws, L.hist), static_cast<hipStream_t>(stream)));
}

moe_status_t moe_grouped_ffn(const moe_config_t* cfg, const int32_t* expert_offsets, const void* x_perm,
                             const void* x_perm_scale, const moe_weights_t* experts, void* y_perm, void* ws,
                             size_t ws_bytes, void* stream) {
  moe_status_t s = check_common(cfg, ws, ws_bytes);
  if (s != MOE_OK || cfg->num_tokens == 0) return s;
  if (!expert_offsets || !x_perm || !y_perm || !weights_ok(*cfg, experts)) return MOE_ERR_INVALID_ARGUMENT;
  if (act_scaled(*cfg) && !x_perm_scale) return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = layout(*cfg);
  FfnScratch sc{at<int32_t>(ws, L.tiles_l), at<int32_t>(ws, L.tiles_s), at<void>(ws, L.h), at<void>(ws, L.h_scale)};
  return to_status(launch_grouped_ffn(*cfg, expert_offsets, x_perm, x_perm_scale, nullptr, *experts, y_perm, sc,
                                      static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(const moe_config_t* cfg, const void* y_perm, const int32_t* pair_pos, const float* topk_w,
                         const void* x, const moe_weights_t* shared, void* out, void* ws, size_t ws_bytes,
                         void* stream) {
  moe_status_t s = check_common(cfg, ws, ws_bytes);
  if (s != MOE_OK || cfg->num_tokens == 0) return s;
  if (!y_perm || !pair_pos || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->num_shared > 0 && (!x || !shared || !shared->w13 || !shared->w2)) return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = layout(*cfg);
  return to_status(launch_combine(*cfg, y_perm, pair_pos, topk_w, x, shared, nullptr, out, at<void>(ws, L.h_shared),
                                  at<float>(ws, L.sh_out), at<float>(ws, L.sh_part), static_cast<hipStream_t>(stream)));
}

moe_status_t moe_forward(const moe_config_t* cfg, const void* x, const float* gate_w, const float* bias,
                         const moe_weights_t* experts, const moe_weights_t* shared, void* out, int32_t* topk_idx_out,
                         float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t s = check_common(cfg, ws, ws_bytes);
  if (s != MOE_OK || cfg->num_tokens == 0) return s;
  if (!x || !gate_w || !bias || !out || !weights_ok(*cfg, experts)) return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->num_shared > 0 && (!shared || !shared->w13 || !shared->w2)) return MOE_ERR_INVALID_ARGUMENT;
  return to_status(forward_impl(*cfg, x, nullptr, gate_w, bias, experts, shared, out, topk_idx_out, topk_w_out, ws,
                                static_cast<hipStream_t>(stream)));
}

moe_status_t moe_rmsnorm(const moe_config_t* cfg, const void* resid, const float* norm_w, float eps, void* x,
                         void* stream) {
  if (!valid_config(cfg)) return MOE_ERR_INVALID_ARGUMENT;
  if (!supported_shape(cfg)) return MOE_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f && eps <= 3.0e38f)) return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!resid || !norm_w || !x || resid == x) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(resid) || !aligned16(norm_w) || !aligned16(x)) return MOE_ERR_INVALID_ARGUMENT;
  return to_status(launch_rmsnorm(*cfg, resid, norm_w, eps, x, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_forward_residual(const moe_config_t* cfg, const void* resid, const float* norm_w, float eps,
                                  const float* gate_w, const float* bias, const moe_weights_t* experts,
                                  const moe_weights_t* shared, void* out, int32_t* topk_idx_out, float* topk_w_out,
                                  void* ws, size_t ws_bytes, void* stream) {
  moe_status_t s = check_common(cfg, ws, ws_bytes);
  if (s != MOE_OK) return s;
  if (!(eps >= 0.0f && eps <= 3.0e38f)) return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->num_tokens == 0) return MOE_OK;
  if (!resid || !norm_w || !gate_w || !bias || !out || !weights_ok(*cfg, experts)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(resid) || !aligned16(norm_w) || !aligned16(out)) return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->num_shared > 0 && (!shared || !shared->w13 || !shared->w2)) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* xn = at<void>(ws, layout(*cfg).xn);
  hipError_t e = launch_rmsnorm(*cfg, resid, norm_w, eps, xn, st);
  if (e == hipSuccess)
    e = forward_impl(*cfg, xn, resid, gate_w, bias, experts, shared, out, topk_idx_out, topk_w_out, ws, st);
  return to_status(e);
}

moe_status_t moe_convert_mxfp4_to_fp8(int64_t rows, int32_t row_len, const void* w_fp4, const void* w_e8m0,
                                      void* w_fp8, float* w_fp8_scale, int32_t* inexact_blocks, void* stream) {
  if (rows < 0 || row_len <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (rows % 128 != 0 || row_len % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!w_fp4 || !w_e8m0 || !w_fp8 || !w_fp8_scale) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(w_fp4) || !aligned16(w_fp8) || !aligned16(w_fp8_scale) ||
      (reinterpret_cast<uintptr_t>(w_e8m0) & 15) || (reinterpret_cast<uintptr_t>(inexact_blocks) & 3))
    return MOE_ERR_INVALID_ARGUMENT;
  if (rows / 128 > 65535) return MOE_ERR_UNSUPPORTED;
  return to_status(launch_mxfp4_to_fp8(rows, row_len, w_fp4, w_e8m0, w_fp8, w_fp8_scale, inexact_blocks,
                                       static_cast<hipStream_t>(stream)));
}

moe_status_t moe_pack_fp4_scales(int32_t recipe, int64_t rows, int32_t row_len, const void* src, void* dst,
                                 void* stream) {
  if (recipe != MOE_RECIPE_MXFP4 && recipe != MOE_RECIPE_NVFP4) return MOE_ERR_INVALID_ARGUMENT;
  if (rows < 0 || row_len <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (rows % 32 != 0 || row_len % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t bytes = rows * (row_len / (recipe == MOE_RECIPE_MXFP4 ? 32 : 16));
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return MOE_ERR_INVALID_ARGUMENT;   // overlapping buffers
  return to_status(launch_pack_fp4_scales(recipe, rows, row_len, src, dst, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
