// Host entry of the routed expert FFN: workspace layout, launch plan and
// the sequence of kernels on the caller's stream (no host synchronisation).
//
//   project V x (gate/up) + x exponents -> gate/up + SwiGLU (h with block
//   exponents) -> project V_down h + h renormalised per pair -> down
//   (gate-scaled split-K partials) -> combine (undoes the h exponent)
#include "common.hpp"
#include "ffn.hpp"
#include "route.hpp"
#include "layer.hpp"

namespace moeq {

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Ws {
  size_t zp_gu, zp_d, zsh, dlead, h, hblk, hn, hexp, hexpf, xexp, xn, ypart, total;
  int ks_gu, ks_d;
};

// Kernel path of one call.  Tiled: on average at least tiled_min_pairs per
// expert (below that, streaming the weights once per 32-token chunk is as
// fast or faster on a Mixtral-sized layer), shapes the tiled kernels cover
// (H a multiple of 256, 32-bit element offsets of the activation rows and
// byte offsets of a block's codes, z rows that fit one activation buffer);
// weight streaming otherwise.  INT and bit-plane blocks alike.
static bool tiled_fits(const moeq_layer *L, int T, int k) {
  const LayerDims &D = L->dims;
  const int64_t P = (int64_t)T * k;
  const int RZ = (D.r + 31) / 32 * 32 + (D.rs + 31) / 32 * 32;
  return D.H % 256 == 0 && D.I % kTileK == 0 && (int64_t)D.H * D.I / 2 < (1ll << 31) &&
         (int64_t)T * D.H < (1ll << 31) && P * D.I < (1ll << 31) && 2 * RZ <= kTileK + 8;
}

// Average pairs per expert from which the tiled path is faster: about 96
// for int4, measured on the Mixtral-sized layer (E = 8, k = 2, I = 14336:
// T = 384) and on the fine-grained one (E = 64, k = 6, I = 1408: T = 1024);
// 384 for int3 on the Mixtral-sized layer (T = 1536), whose fields cost the
// tiled decode more; layers with any block below 4 bits take the larger
// figure.  Bit-plane layers: 192, between the points measured on the
// 128-expert layer (k = 8, H = 2048, I = 768, q in {2, 3, 4}): streaming
// 6% faster at 128 pairs per expert (T = 2048), tiled 5% faster at 256.
static int64_t tiled_min_pairs(const moeq_layer *L) {
  if (L->dims.fmt == MOEQ_FMT_BITPLANE) return 192;
  for (uint8_t b : L->bits)
    if (b != 4) return 384;
  return 96;
}

// Fewest gate/up workgroups (token tiles x 128-row tiles of I) for which the
// tiled path is taken: below one per CU its grid leaves the chip idle (the
// 8-expert layer with H = 256, I = 512 streams faster at every batch up to
// 384 pairs per expert, where its tiled grid has 124 workgroups).
constexpr int64_t kTiledMinGrid = 256;

static int pick_path(const moeq_layer *L, int T, int k, const moeq_ffn_options *o) {
  const int want = o ? o->path : MOEQ_PATH_AUTO;
  if (want == MOEQ_PATH_TILED) return tiled_fits(L, T, k) ? MOEQ_PATH_TILED : -1;
  if (want == MOEQ_PATH_STREAM) return MOEQ_PATH_STREAM;
  if (want != MOEQ_PATH_AUTO) return -1;
  const int64_t P = (int64_t)T * k;
  const int64_t grid = (int64_t)max_chunks(L->dims.E, T, k, kTiledM) * (L->dims.I / kTileK);
  return (tiled_fits(L, T, k) && P >= tiled_min_pairs(L) * L->dims.E && grid >= kTiledMinGrid)
             ? MOEQ_PATH_TILED : MOEQ_PATH_STREAM;
}

static int pick_splits(const moeq_layer *L, int T, int k, const moeq_ffn_options *o) {
  if (pick_path(L, T, k, o) == MOEQ_PATH_TILED) return 1;
  if (o && o->split_k > 0) return o->split_k;
  const int P = T * k;
  const int n_g4 = (L->dims.I / kTileK + 3) / 4;
  // few tokens: split the long down-projection K for more waves in flight
  int s = P <= 256 ? 4 : 1;
  return std::max(1, std::min(s, n_g4));
}

// K splits of a low-rank projection over K columns: few tokens leave few
// workgroups, so cut K into ~1024-column pieces; many tokens need none.
static int pick_ks(int P, int K) {
  if (P > 256) return 1;
  return std::max(1, std::min(16, K / 1024));
}

// The down projection in wave tiles (lowrank_project_kernel, WT): many
// pairs, no shared factors, at most four 16-column jobs, and a K long
// enough to split over the grid.  Its K splits make about 1024 workgroups.
static bool wave_tiles(const moeq_layer *L, int64_t P) {
  const int Rp = (L->dims.r + 31) / 32 * 32;
  return P > 256 && L->dims.rs == 0 && Rp > 0 && Rp / 16 <= 4 && L->dims.I >= 4096;
}
static int wave_tile_ks(const moeq_layer *L, int64_t P) {
  const int64_t tiles = P / 64 + L->dims.E;
  return (int)std::max<int64_t>(1, std::min<int64_t>({(1024 + tiles - 1) / tiles, 8, L->dims.I / 1024}));
}

static int hblk_stride(const moeq_layer *L) { return (L->dims.I / 64 + 15) / 16 * 16; }

// z_tok: the gate/up projection covers every (token, expert) pair (the
// fused routing path) instead of the routed pairs.
static Ws ws_plan(const moeq_layer *L, int T, int k, int splits, bool z_tok = false) {
  const int64_t P = (int64_t)T * k;
  const int64_t PZ = z_tok ? (int64_t)T * L->dims.E : P;
  const int Rp = (L->dims.r + 31) / 32 * 32, Rsp = (L->dims.rs + 31) / 32 * 32;
  const int RZ = Rp + Rsp;
  Ws w;
  w.ks_gu = pick_ks((int)PZ, L->dims.H);
  w.ks_d = wave_tiles(L, P) ? wave_tile_ks(L, P) : pick_ks((int)P, L->dims.I);
  size_t off = 0;
  w.zp_gu = off; off = al256(off + (size_t)w.ks_gu * PZ * 2 * RZ * 4);
  w.zp_d = off; off = al256(off + (size_t)w.ks_d * P * RZ * 4);
  w.zsh = off; off = al256(off + (size_t)w.ks_d * P * k * Rsp * 4);
  w.dlead = off; off = al256(off + (Rsp ? (size_t)P * 4 : 0));
  w.h = off; off = al256(off + (size_t)P * L->dims.I * 2);
  w.hblk = off; off = al256(off + (size_t)P * hblk_stride(L));
  w.hn = off; off = al256(off + (size_t)P * L->dims.I * 2);
  w.hexp = off; off = al256(off + (size_t)P * 4);
  w.hexpf = off; off = al256(off + (size_t)P * 4);
  w.xexp = off; off = al256(off + (size_t)T * 4);
  w.xn = off; off = al256(off + (size_t)T * L->dims.H * 2);
  w.ypart = off; off = al256(off + (size_t)splits * P * L->dims.H * 4);
  w.total = off;
  return w;
}

// Argument checks, workspace layout and the argument block of one call.
static moeq_status ffn_setup(const moeq_layer *L, const uint16_t *x, int32_t T, int32_t k, const moeq_routing *r,
                             int32_t n_comp, void *y, int32_t y_dtype, void *ws, size_t ws_bytes,
                             const moeq_ffn_options *opts, bool z_tok, FfnArgs *out, int *path_out) {
  if (!L || !r) return fail(MOEQ_ERR_INVALID, "expert_ffn: null layer or routing");
  const LayerDims &D = L->dims;
  if (T < 0 || k < 1 || k > D.E) return fail(MOEQ_ERR_INVALID, "expert_ffn: T=%d k=%d invalid for E=%d", T, k, D.E);
  if (n_comp < 0 || n_comp > k) return fail(MOEQ_ERR_INVALID, "expert_ffn: n_comp=%d not in 0..%d", n_comp, k);
  if (y_dtype != MOEQ_F16 && y_dtype != MOEQ_F32) return fail(MOEQ_ERR_INVALID, "expert_ffn: bad y_dtype %d", y_dtype);
  const int path = pick_path(L, T, k, opts);
  if (path < 0)
    return fail(MOEQ_ERR_UNSUPPORTED, "expert_ffn: path %d not available for this layer and batch",
                opts ? opts->path : 0);
  if (opts && (opts->split_k < 0 || opts->split_k > 64)) return fail(MOEQ_ERR_INVALID, "expert_ffn: split_k=%d not in 0..64", opts->split_k);
  *path_out = path;
  if (T == 0) return MOEQ_OK;
  if (!x || !y || !r->topk_gates || !r->expert_offsets || !r->sorted_pairs || !r->pair_pos)
    return fail(MOEQ_ERR_INVALID, "expert_ffn: null pointer");
  if (D.rs > 0 && n_comp > 0 && !r->topk_ids)
    return fail(MOEQ_ERR_INVALID, "expert_ffn: a layer with shared factors needs the routing's topk_ids");
  if (D.rs > 0 && n_comp > 32)
    return fail(MOEQ_ERR_UNSUPPORTED, "expert_ffn: shared factors with n_comp=%d > 32 compensated slots", n_comp);
  const int splits = pick_splits(L, T, k, opts);
  const Ws w = ws_plan(L, T, k, splits, z_tok);
  if (!ws || ws_bytes < w.total)
    return fail(MOEQ_ERR_WORKSPACE, "expert_ffn: workspace has %zu bytes, needs %zu", ws_bytes, w.total);

  uint8_t *wb = static_cast<uint8_t *>(ws);
  FfnArgs &a = *out;
  a.desc = L->d_desc;
  a.offsets = r->expert_offsets;
  a.sorted_pairs = r->sorted_pairs;
  a.x = x;
  a.gates = r->topk_gates;
  a.pair_pos = r->pair_pos;
  a.ids = r->topk_ids;
  a.share = D.rs > 0 ? D.share : 1;
  a.E = D.E; a.H = D.H; a.I = D.I; a.k = k; a.T = T; a.n_comp = n_comp;
  a.r = D.r; a.rs = D.rs;
  a.Rp = (D.r + 31) / 32 * 32; a.Rsp = (D.rs + 31) / 32 * 32; a.RZ = a.Rp + a.Rsp;
  a.comp_on = (n_comp > 0 && a.RZ > 0) ? 1 : 0;
  a.zp_gu = reinterpret_cast<float *>(wb + w.zp_gu);
  a.zp_d = reinterpret_cast<float *>(wb + w.zp_d);
  a.zsh = reinterpret_cast<float *>(wb + w.zsh);
  a.dlead = reinterpret_cast<int32_t *>(wb + w.dlead);
  a.ks_stride_sh = (int64_t)T * k * k * ((D.rs + 31) / 32 * 32);
  a.z_tok = z_tok ? 1 : 0;
  a.ks_gu = w.ks_gu;
  a.ks_d = w.ks_d;
  a.wt = wave_tiles(L, (int64_t)T * k) ? 1 : 0;
  a.ks_stride_gu = (int64_t)T * (z_tok ? D.E : k) * 2 * a.RZ;
  a.ks_stride_d = (int64_t)T * k * a.RZ;
  a.h = reinterpret_cast<uint16_t *>(wb + w.h);
  a.hblk = reinterpret_cast<int8_t *>(wb + w.hblk);
  a.hblk_stride = hblk_stride(L);
  a.hn = reinterpret_cast<uint16_t *>(wb + w.hn);
  a.hexp = reinterpret_cast<int32_t *>(wb + w.hexp);
  a.hexpf = reinterpret_cast<int32_t *>(wb + w.hexpf);
  a.xexp = reinterpret_cast<int32_t *>(wb + w.xexp);
  a.xn = reinterpret_cast<uint16_t *>(wb + w.xn);
  a.ypart = reinterpret_cast<float *>(wb + w.ypart);
  a.splits = splits;
  a.P = T * k;
  a.G = D.G;
  a.fmt = D.fmt;
  a.nsub_max = std::max(1, std::min(kMT, T) / 16 + (std::min(kMT, T) % 16 ? 1 : 0));
  return MOEQ_OK;
}

// First launch: x exponents and the normalised x * 2^K that the gate/up
// kernels read, with the gate/up projection when there is one (of the
// routed pairs, or with z_tok of every (token, expert) pair).
static void ffn_front(const FfnArgs &a, hipStream_t stream) {
  if (a.comp_on) {
    prof_begin("lowrank_project_gu", stream);
    launch_lowrank_project(a, a.z_tok ? 2 : 0, 2 * a.RZ / 16, stream);
    prof_end("lowrank_project_gu", stream);
  } else {
    prof_begin("xexp", stream);
    launch_xexp(a, stream);
    prof_end("xexp", stream);
  }
}

// The rest of the call, after routing and ffn_front.
static moeq_status ffn_rest(const FfnArgs &a, int path, void *y, int32_t y_dtype, hipStream_t stream) {
  const int mc = max_chunks(a.E, a.T, a.k);
  const bool tiled = path == MOEQ_PATH_TILED;
  const int mt = tiled ? max_chunks(a.E, a.T, a.k, kTiledM) : 0;     // token tiles of the tiled path
  if (tiled) {
    prof_begin("gateup_tiled", stream);
    launch_tiled_gateup(a, (mt * (a.I / kTileK) + 7) / 8 * 8, stream);
    prof_end("gateup_tiled", stream);
  } else {
    prof_begin("gateup_stream", stream);
    launch_gateup_stream(a, mc * (a.I / 64), stream);
    prof_end("gateup_stream", stream);
  }
  // h renormalised to one exponent per pair (with the down projection when
  // there is one)
  if (a.comp_on) {
    prof_begin("lowrank_project_down", stream);
    launch_lowrank_project(a, 1, a.RZ / 16, stream);
    prof_end("lowrank_project_down", stream);
  } else {
    prof_begin("hnorm", stream);
    launch_hnorm(a, stream);
    prof_end("hnorm", stream);
  }
  if (tiled) {
    prof_begin("down_tiled", stream);
    launch_tiled_down(a, (mt * (a.H / 256) + 7) / 8 * 8, stream);
    prof_end("down_tiled", stream);
  } else {
    prof_begin("down_stream", stream);
    launch_down_stream(a, mc * (a.H / 128) * a.splits, stream);
    prof_end("down_stream", stream);
  }
  prof_begin("combine", stream);
  launch_combine(a, y, y_dtype == MOEQ_F32, stream);
  prof_end("combine", stream);
  return check_launch("expert_ffn");
}

// The fused routing path serves decode-sized batches whose expert count is
// small against k (the projection of every (token, expert) pair then costs
// little more than that of the routed pairs) on the weight-streaming path.
static bool fusable(const moeq_layer *L, int T, int k, const moeq_ffn_options *opts) {
  return T >= 1 && T <= kRouteTokens && L->dims.E <= kMaxE && L->dims.E <= 4 * k && pick_path(L, T, k, opts) == MOEQ_PATH_STREAM;
}

}  // namespace moeq

using namespace moeq;

MOEQ_API moeq_status moeq_ffn_workspace_size(const moeq_layer *L, int32_t T, int32_t k,
                                             const moeq_ffn_options *opts, size_t *bytes) {
  if (!L || !bytes) return fail(MOEQ_ERR_INVALID, "ffn_workspace_size: null argument");
  if (T < 0 || k < 1 || k > L->dims.E) return fail(MOEQ_ERR_INVALID, "ffn_workspace_size: T=%d k=%d invalid", T, k);
  if (opts && (opts->split_k < 0 || opts->split_k > 64)) return fail(MOEQ_ERR_INVALID, "ffn_workspace_size: split_k=%d not in 0..64", opts->split_k);
  *bytes = ws_plan(L, T, k, pick_splits(L, T, k, opts)).total;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_expert_ffn(const moeq_layer *L, const uint16_t *x, int32_t T, int32_t k,
                                     const moeq_routing *r, int32_t n_comp, void *y, int32_t y_dtype,
                                     void *ws, size_t ws_bytes, const moeq_ffn_options *opts,
                                     hipStream_t stream) {
  FfnArgs a;
  int path = 0;
  moeq_status st = ffn_setup(L, x, T, k, r, n_comp, y, y_dtype, ws, ws_bytes, opts, false, &a, &path);
  if (st != MOEQ_OK || T == 0) return st;
  ffn_front(a, stream);
  return ffn_rest(a, path, y, y_dtype, stream);
}

// Unfused calls: the FFN's workspace, then (long batches) the routing's.
MOEQ_API moeq_status moeq_forward_workspace_size(const moeq_layer *L, int32_t T, int32_t k,
                                                 const moeq_ffn_options *opts, size_t *bytes) {
  moeq_status st = moeq_ffn_workspace_size(L, T, k, opts, bytes);
  if (st != MOEQ_OK) return st;
  if (fusable(L, T, k, opts)) {
    *bytes = ws_plan(L, T, k, pick_splits(L, T, k, opts), true).total;
  } else {
    size_t rb = 0;
    st = moeq_route_workspace_size(T, L->dims.E, k, &rb);
    if (st != MOEQ_OK) return st;
    if (rb) *bytes = al256(*bytes) + rb;
  }
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_moe_forward(const moeq_layer *L, const float *logits, const uint16_t *x, int32_t T,
                                      int32_t k, int32_t n_comp, const moeq_routing *r, void *y, int32_t y_dtype,
                                      void *ws, size_t ws_bytes, const moeq_ffn_options *opts, hipStream_t stream) {
  if (!L || !r) return fail(MOEQ_ERR_INVALID, "moe_forward: null layer or routing");
  if (!fusable(L, T, k, opts)) {
    // routing (into the end of ws when it needs a workspace), then the
    // expert FFN
    size_t fb = 0, rb = 0;
    moeq_status st = moeq_ffn_workspace_size(L, T, k, opts, &fb);
    if (st != MOEQ_OK) return st;
    st = moeq_route_workspace_size(T, L->dims.E, k, &rb);
    if (st != MOEQ_OK) return st;
    void *rws = nullptr;
    if (rb) {
      if (!ws || ws_bytes < al256(fb) + rb)
        return fail(MOEQ_ERR_WORKSPACE, "moe_forward: workspace has %zu bytes, needs %zu", ws_bytes, al256(fb) + rb);
      rws = static_cast<uint8_t *>(ws) + al256(fb);
    }
    st = moeq_route(logits, T, L->dims.E, k, r, rws, rb, stream);
    if (st != MOEQ_OK) return st;
    return moeq_expert_ffn(L, x, T, k, r, n_comp, y, y_dtype, ws, ws_bytes, opts, stream);
  }
  FfnArgs a;
  int path = 0;
  moeq_status st = ffn_setup(L, x, T, k, r, n_comp, y, y_dtype, ws, ws_bytes, opts, true, &a, &path);
  if (st != MOEQ_OK) return st;
  if (!logits || !r->topk_ids) return fail(MOEQ_ERR_INVALID, "moe_forward: null pointer");
  // routing, x exponents and every pair's gate/up projection in one launch
  const RouteOut ro{logits, r->topk_ids, r->topk_gates, r->expert_offsets, r->sorted_pairs, r->pair_pos};
  prof_begin("front_routed", stream);
  launch_front_routed(a, ro, stream);
  prof_end("front_routed", stream);
  return ffn_rest(a, path, y, y_dtype, stream);
}
