// Host entry of the routed expert FFN: workspace layout, launch plan and
// the sequence of kernels on the caller's stream (no host synchronisation).
//
//   project V x (gate/up) -> gate/up stream + SwiGLU -> project V_down h
//   -> down stream (split-K partials) -> gate-weighted combine
#include "common.hpp"
#include "ffn.hpp"
#include "layer.hpp"

namespace moeq {

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Ws {
  size_t zp_gu, zp_d, h, ypart, total;
  int ks_gu, ks_d;
};

// Kernel path of one call.  Tiled: INT blocks, on average at least
// tiled_min_pairs per expert (below that, streaming the weights once per
// 32-token chunk is as fast or faster on a Mixtral-sized layer), shapes the tiled kernels cover (H a multiple of 256, 32-bit
// element offsets of the activation rows, z rows that fit one activation
// buffer); weight streaming otherwise.
static bool tiled_fits(const moeq_layer *L, int T, int k) {
  const LayerDims &D = L->dims;
  const int64_t P = (int64_t)T * k;
  const int RZ = (D.r + 31) / 32 * 32 + (D.rs + 31) / 32 * 32;
  return D.fmt == MOEQ_FMT_INT && D.H % 256 == 0 && D.I % kTileK == 0 &&
         (int64_t)T * D.H < (1ll << 31) && P * D.I < (1ll << 31) && 2 * RZ <= kTileK + 8;
}

// Average pairs per expert from which the tiled path is faster, measured on
// the Mixtral-sized layer (E = 8, k = 2): about 96 for int4 (T = 384) and
// 384 for int3 (T = 1536), whose fields cost the tiled decode more; layers
// with any block below 4 bits take the larger figure.
static int64_t tiled_min_pairs(const moeq_layer *L) {
  for (uint8_t b : L->bits)
    if (b != 4) return 384;
  return 96;
}

static int pick_path(const moeq_layer *L, int T, int k, const moeq_ffn_options *o) {
  const int want = o ? o->path : MOEQ_PATH_AUTO;
  if (want == MOEQ_PATH_TILED) return tiled_fits(L, T, k) ? MOEQ_PATH_TILED : -1;
  if (want == MOEQ_PATH_STREAM) return MOEQ_PATH_STREAM;
  if (want != MOEQ_PATH_AUTO) return -1;
  const int64_t P = (int64_t)T * k;
  return (tiled_fits(L, T, k) && P >= tiled_min_pairs(L) * L->dims.E) ? MOEQ_PATH_TILED : MOEQ_PATH_STREAM;
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

static Ws ws_plan(const moeq_layer *L, int T, int k, int splits) {
  const int64_t P = (int64_t)T * k;
  const int Rp = (L->dims.r + 31) / 32 * 32, Rsp = (L->dims.rs + 31) / 32 * 32;
  const int RZ = Rp + Rsp;
  Ws w;
  w.ks_gu = pick_ks((int)P, L->dims.H);
  w.ks_d = pick_ks((int)P, L->dims.I);
  size_t off = 0;
  w.zp_gu = off; off = al256(off + (size_t)w.ks_gu * P * 2 * RZ * 4);
  w.zp_d = off; off = al256(off + (size_t)w.ks_d * P * RZ * 4);
  w.h = off; off = al256(off + (size_t)P * L->dims.I * 2);
  w.ypart = off; off = al256(off + (size_t)splits * P * L->dims.H * 4);
  w.total = off;
  return w;
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
  if (T == 0) return MOEQ_OK;
  if (!x || !y || !r->topk_gates || !r->expert_offsets || !r->sorted_pairs || !r->pair_pos)
    return fail(MOEQ_ERR_INVALID, "expert_ffn: null pointer");
  const int splits = pick_splits(L, T, k, opts);
  const Ws w = ws_plan(L, T, k, splits);
  if (!ws || ws_bytes < w.total)
    return fail(MOEQ_ERR_WORKSPACE, "expert_ffn: workspace has %zu bytes, needs %zu", ws_bytes, w.total);

  uint8_t *wb = static_cast<uint8_t *>(ws);
  FfnArgs a;
  a.desc = L->d_desc;
  a.offsets = r->expert_offsets;
  a.sorted_pairs = r->sorted_pairs;
  a.x = x;
  a.gates = r->topk_gates;
  a.pair_pos = r->pair_pos;
  a.E = D.E; a.H = D.H; a.I = D.I; a.k = k; a.T = T; a.n_comp = n_comp;
  a.r = D.r; a.rs = D.rs;
  a.Rp = (D.r + 31) / 32 * 32; a.Rsp = (D.rs + 31) / 32 * 32; a.RZ = a.Rp + a.Rsp;
  a.comp_on = (n_comp > 0 && a.RZ > 0) ? 1 : 0;
  a.zp_gu = reinterpret_cast<float *>(wb + w.zp_gu);
  a.zp_d = reinterpret_cast<float *>(wb + w.zp_d);
  a.ks_gu = w.ks_gu;
  a.ks_d = w.ks_d;
  a.ks_stride_gu = (int64_t)T * k * 2 * a.RZ;
  a.ks_stride_d = (int64_t)T * k * a.RZ;
  a.h = reinterpret_cast<uint16_t *>(wb + w.h);
  a.ypart = reinterpret_cast<float *>(wb + w.ypart);
  a.splits = splits;
  a.P = T * k;

  const int mc = max_chunks(D.E, T, k);
  a.G = D.G;
  a.fmt = D.fmt;
  a.nsub_max = std::max(1, std::min(kMT, T) / 16 + (std::min(kMT, T) % 16 ? 1 : 0));
  if (a.comp_on) {
    prof_begin("lowrank_project_gu", stream);
    launch_lowrank_project(a, 0, dim3(mc * kSubPerChunk, 2 * a.RZ / 16), stream);
    prof_end("lowrank_project_gu", stream);
  }
  const bool tiled = path == MOEQ_PATH_TILED;
  const int mt = tiled ? max_chunks(D.E, T, k, kTiledM) : 0;     // token tiles of the tiled path
  if (tiled) {
    prof_begin("gateup_tiled", stream);
    launch_tiled_gateup(a, (mt * (D.I / kTileK) + 7) / 8 * 8, stream);
    prof_end("gateup_tiled", stream);
  } else {
    prof_begin("gateup_stream", stream);
    launch_gateup_stream(a, mc * (D.I / 64), stream);
    prof_end("gateup_stream", stream);
  }
  if (a.comp_on) {
    prof_begin("lowrank_project_down", stream);
    launch_lowrank_project(a, 1, dim3(mc * kSubPerChunk, a.RZ / 16), stream);
    prof_end("lowrank_project_down", stream);
  }
  if (tiled) {
    prof_begin("down_tiled", stream);
    launch_tiled_down(a, (mt * (D.H / 256) + 7) / 8 * 8, stream);
    prof_end("down_tiled", stream);
  } else {
    prof_begin("down_stream", stream);
    launch_down_stream(a, mc * (D.H / 128) * splits, stream);
    prof_end("down_stream", stream);
  }
  prof_begin("combine", stream);
  launch_combine(a, y, y_dtype == MOEQ_F32, stream);
  prof_end("combine", stream);
  return check_launch("expert_ffn");
}
