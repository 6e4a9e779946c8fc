// Host-side checks of the C-ABI library under AddressSanitizer and UBSan (host code
// only; nothing here launches a kernel or needs a GPU):
//   - the workspace layout: every region 256-byte aligned, in order, inside
//     moe_workspace_bytes; the gate's scratch inside its region;
//   - the tile-list bounds that size the workspace: the counts the device
//     builder writes, for adversarial per-expert row counts, stay within them;
//   - argument validation: each entry point's error for each bad argument,
//     returned before anything is enqueued;
//   - the GEMM kernels' block -> tile map (xcd_tile, tile_coords) is a bijection.
// The translation unit includes the library's API source, so its internal layout
// and plan functions are the ones under test.
#include "../../mixture_experts_amd/csrc/moe_api.hip"

#include <cmath>
#include <cstdio>
#include <random>
#include <string>

namespace {

int failures = 0;
#define CHECK(cond, ...)                                           \
  do {                                                             \
    if (!(cond)) {                                                 \
      ++failures;                                                  \
      std::printf("FAIL line %d: %s: ", __LINE__, #cond);          \
      std::printf(__VA_ARGS__);                                    \
      std::printf("\n");                                           \
    }                                                              \
  } while (0)

moe_config_t make(int T, int H, int E, int k, int I, int S, int SI, int ng, int tg, int recipe, int func = 0) {
  moe_config_t c{};
  c.num_tokens = T;
  c.hidden = H;
  c.num_experts = E;
  c.top_k = k;
  c.intermediate = I;
  c.num_shared = S;
  c.shared_intermediate = SI;
  c.n_group = ng;
  c.topk_group = tg;
  c.score_func = func;
  c.norm_topk_prob = 1;
  c.routed_scaling_factor = 2.5f;
  c.recipe = recipe;
  c.swiglu_limit = 0.0f;
  return c;
}

// Tile counts the device builder writes for per-expert row counts m (as ffn_misc.hip's
// build_tiles2 does: experts with >= thresh rows into bm_l-row tiles, the others into
// bm_s-row tiles).
void tile_counts(const FfnPlan& p, const std::vector<int64_t>& m, int64_t& nl, int64_t& ns) {
  nl = ns = 0;
  for (int64_t r : m) {
    if (r >= p.thresh) nl += (r + p.bm_l - 1) / p.bm_l;
    else ns += (r + p.bm_s - 1) / p.bm_s;
  }
}

// Row counts: each expert takes at most T rows (a token picks an expert once) and
// they sum to T * k.
std::vector<std::vector<int64_t>> loads(const moe_config_t& c, std::mt19937_64& rng) {
  const int64_t T = c.num_tokens, E = c.num_experts, P = T * c.top_k;
  std::vector<std::vector<int64_t>> out;
  auto fill = [&](int64_t per) {                    // as many experts as possible with `per` rows
    std::vector<int64_t> m(E, 0);
    int64_t left = P;
    for (int64_t e = 0; e < E && left > 0; ++e) {
      m[e] = std::min<int64_t>({per, T, left});
      left -= m[e];
    }
    for (int64_t e = 0; e < E && left > 0; ++e) {   // the rest where room is left
      const int64_t add = std::min<int64_t>(T - m[e], left);
      m[e] += add;
      left -= add;
    }
    out.push_back(m);
  };
  const FfnPlan p = ffn_plan(c);
  for (int64_t per : {int64_t(1), int64_t(p.bm_s + 1), int64_t(p.thresh - 1), int64_t(p.thresh),
                      int64_t(p.bm_l + 1), int64_t(2 * p.bm_l + 1), (P + E - 1) / E, T}) {
    if (per >= 1) fill(per);
  }
  for (int rep = 0; rep < 20; ++rep) {              // random: Dirichlet-like shares, clipped at T
    std::vector<double> w(E);
    std::exponential_distribution<double> ex(1.0);
    double s = 0;
    for (auto& v : w) s += (v = std::pow(ex(rng), 1.0 + rep % 4));
    std::vector<int64_t> m(E, 0);
    int64_t left = P;
    for (int64_t e = 0; e < E; ++e) {
      m[e] = std::min<int64_t>({T, left, int64_t(w[e] / s * P)});
      left -= m[e];
    }
    for (int64_t e = 0; e < E && left > 0; ++e) {
      const int64_t add = std::min<int64_t>(T - m[e], left);
      m[e] += add;
      left -= add;
    }
    out.push_back(m);
  }
  return out;
}

void check_layout(const moe_config_t& c, std::mt19937_64& rng) {
  const Layout L = layout(c);
  const size_t offs[] = {L.route, L.hist, L.tiles_l, L.tiles_s, L.h, L.h_scale, L.h_shared, L.sh_out, L.sh_part,
                         L.idx, L.w, L.offsets, L.sorted, L.pos, L.xq, L.xq_scale, L.y_perm, L.xn, L.total};
  const int n = int(sizeof(offs) / sizeof(offs[0]));
  for (int i = 0; i < n; ++i) CHECK(offs[i] % 256 == 0, "T=%d region %d at %zu", c.num_tokens, i, offs[i]);
  for (int i = 0; i + 1 < n; ++i) CHECK(offs[i] < offs[i + 1], "T=%d regions %d, %d out of order", c.num_tokens, i, i + 1);
  CHECK(L.total == moe_workspace_bytes(&c), "T=%d total %zu vs %zu", c.num_tokens, L.total, moe_workspace_bytes(&c));
  CHECK(route_workspace_bytes(c) <= L.hist - L.route, "T=%d gate scratch %zu > region %zu", c.num_tokens,
        route_workspace_bytes(c), L.hist - L.route);
  const FfnPlan p = ffn_plan(c);
  CHECK(size_t(2 * int64_t(p.max_l) + 1) * 4 <= L.tiles_s - L.tiles_l, "T=%d list L region", c.num_tokens);
  CHECK(size_t(2 * int64_t(p.max_s) + 1) * 4 <= L.h - L.tiles_s, "T=%d list S region", c.num_tokens);
  for (const auto& m : loads(c, rng)) {
    int64_t nl, ns;
    tile_counts(p, m, nl, ns);
    CHECK(nl <= p.max_l, "T=%d E=%d k=%d recipe=%d: %lld large tiles > bound %d", c.num_tokens, c.num_experts, c.top_k,
          c.recipe, (long long)nl, p.max_l);
    CHECK(ns <= p.max_s, "T=%d E=%d k=%d recipe=%d: %lld small tiles > bound %d", c.num_tokens, c.num_experts, c.top_k,
          c.recipe, (long long)ns, p.max_s);
  }
}

// The GEMM kernels' block -> tile map: xcd_tile, then tile_coords, must hit every
// (row tile, column tile) once, for every group size the host picks and ragged
// row-tile counts (a last group with fewer row tiles).
void check_tile_map() {
  for (int ncols : {1, 2, 8, 16, 28, 32, 56})
    for (int nrt = 1; nrt <= 70; ++nrt)
      for (int group : {0, 2, 8}) {
        const int V = nrt * ncols;
        std::vector<int> seen(size_t(V), 0);
        bool ok = true;
        for (int b = 0; b < V; ++b) {
          const int t = xcd_tile(b, V);
          int mt = -1, nt = -1;
          if (t < 0 || t >= V) { ok = false; break; }
          tile_coords(t, V, ncols, group, mt, nt);
          if (mt < 0 || mt >= nrt || nt < 0 || nt >= ncols) { ok = false; break; }
          ++seen[size_t(mt) * ncols + nt];
        }
        for (int v : seen) ok = ok && v == 1;
        CHECK(ok, "ncols=%d row tiles=%d group=%d", ncols, nrt, group);
      }
}

void check_validation() {
  moe_config_t c = make(64, 256, 16, 4, 128, 1, 128, 1, 1, MOE_RECIPE_F32);
  alignas(256) static char ws_small[256];
  const size_t need = moe_workspace_bytes(&c);
  CHECK(need > 0, "workspace size of a valid config");
  char dummy_buf[64];
  void* d = dummy_buf;                                // never dereferenced: every call below fails validation
  int32_t* di = reinterpret_cast<int32_t*>(dummy_buf);
  float* df = reinterpret_cast<float*>(dummy_buf);
  moe_weights_t w{d, nullptr, d, nullptr};
  // null and bad configurations
  CHECK(moe_workspace_bytes(nullptr) == 0, "null config");
  moe_config_t bad = c;
  bad.num_experts = 2000;
  CHECK(moe_workspace_bytes(&bad) == 0, "E > 1024");
  CHECK(moe_route(&bad, d, df, df, di, df, ws_small, sizeof ws_small, nullptr) == MOE_ERR_INVALID_ARGUMENT, "E > 1024");
  bad = c;
  bad.top_k = 0;
  CHECK(moe_forward(&bad, d, df, df, &w, &w, d, di, df, ws_small, sizeof ws_small, nullptr) == MOE_ERR_INVALID_ARGUMENT,
        "k = 0");
  bad = c;
  bad.n_group = 3;                                    // 16 experts in 3 groups
  CHECK(moe_route(&bad, d, df, df, di, df, ws_small, sizeof ws_small, nullptr) == MOE_ERR_INVALID_ARGUMENT, "groups");
  bad = c;
  bad.hidden = 100;                                   // not a multiple of 32
  CHECK(moe_route(&bad, d, df, df, di, df, ws_small, sizeof ws_small, nullptr) == MOE_ERR_UNSUPPORTED, "H = 100");
  // workspace: too small, misaligned, null
  CHECK(moe_route(&c, d, df, df, di, df, ws_small, sizeof ws_small, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL,
        "small workspace");
  CHECK(moe_route(&c, d, df, df, di, df, ws_small + 16, need, nullptr) == MOE_ERR_INVALID_ARGUMENT, "misaligned ws");
  CHECK(moe_route(&c, d, df, df, di, df, nullptr, need, nullptr) == MOE_ERR_INVALID_ARGUMENT, "null ws");
  // T = 0: nothing to do, no launch
  moe_config_t empty = c;
  empty.num_tokens = 0;
  CHECK(moe_forward(&empty, d, df, df, &w, &w, d, di, df, nullptr, 0, nullptr) == MOE_OK, "T = 0");
  CHECK(std::string(moe_status_string(MOE_ERR_UNSUPPORTED)).size() > 0, "status string");
}

}  // namespace

int main() {
  std::mt19937_64 rng(7);
  const int recipes[] = {MOE_RECIPE_F32, MOE_RECIPE_BF16, MOE_RECIPE_FP8_B128, MOE_RECIPE_MXFP4, MOE_RECIPE_NVFP4};
  // the workloads' shapes and a spread of token counts, expert counts and top-k
  for (int rc : recipes) {
    const int H = 7168, I = (rc == MOE_RECIPE_F32) ? 2048 : 2048;
    for (int T : {1, 5, 31, 32, 33, 128, 255, 256, 257, 511, 512, 560, 4096, 8192, 16384}) {
      for (int E : {8, 16, 256, 384, 896, 1024}) {
        for (int k : {1, 4, 8, 16}) {
          if (k > E) continue;
          check_layout(make(T, H, E, k, I, 1, 2048, 1, 1, rc), rng);
        }
      }
    }
    check_layout(make(8192, 7168, 256, 8, 2048, 1, 2048, 8, 4, rc), rng);
    check_layout(make(4096, 7168, 896, 16, 1024, 2, 1024, 1, 1, rc), rng);
  }
  check_validation();
  check_tile_map();
  std::printf("host checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
