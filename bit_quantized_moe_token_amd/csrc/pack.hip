// Packing of a quantized layer into the tiled device layout read by the
// expert kernels, and the debug read-back that uses the kernels' decode.
// Each expert linear block is one "weight page" region (PagedWeight review,
// "What carries the argument"); bit-plane blocks store their four planes
// plane by plane, most significant first, so the q planes a block is
// committed to are the first q regions (Figure 3 caption).
#include <cstring>
#include <new>
#include "common.hpp"
#include "decode.hpp"
#include "layer.hpp"

namespace moeq {

// Code of (row, column) for lane l, pair P = 4j + v, half h of a tile.
__device__ __forceinline__ int tile_col(int t, int l, int P, int h) {
  const int j = P >> 2, v = P & 3;
  return t * kTileK + 32 * j + 8 * (l >> 4) + 2 * v + h;
}

template <int B>
__global__ void __launch_bounds__(256)
pack_int_kernel(const uint8_t *__restrict__ codes, int N, int K, uint8_t *__restrict__ out) {
  const int n_kt = K / kTileK;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(N / kStripRows) * n_kt * 64;
  if (id >= total) return;
  const int l = (int)(id & 63);
  const int t = (int)((id >> 6) % n_kt);
  const int s = (int)((id >> 6) / n_kt);
  const int row = s * kStripRows + (l & 15);
  const uint8_t *src = codes + (int64_t)row * K;
  uint32_t d[4] = {0, 0, 0, 0};
#pragma unroll
  for (int P = 0; P < 16; ++P) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = src[tile_col(t, l, P, h)] & ((1u << B) - 1);
      const Field f = int_field<B>(P);
      if (f.e < 0) {
#pragma unroll
        for (int i = 0; i < 3; ++i) d[i] |= ((c >> i) & 1u) << (16 * h + spare3_bit(i));
      } else {
        d[f.e] |= c << (16 * h + f.s + f.p);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < B; ++e) *reinterpret_cast<uint32_t *>(out + int_word_offset(s, t, l, e, n_kt, B)) = d[e];
}

// Four bit-planes of 4-bit parent codes; plane c goes to region 3 - c.
__global__ void __launch_bounds__(256)
pack_planes_kernel(const uint8_t *__restrict__ codes, int N, int K, uint8_t *__restrict__ out,
                   uint64_t plane_bytes) {
  const int n_kt = K / kTileK;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(N / kStripRows) * n_kt * 64;
  if (id >= total) return;
  const int l = (int)(id & 63);
  const int t = (int)((id >> 6) % n_kt);
  const int s = (int)((id >> 6) / n_kt);
  const int row = s * kStripRows + (l & 15);
  const uint8_t *src = codes + (int64_t)row * K;
  uint32_t pl[4] = {0, 0, 0, 0};
#pragma unroll
  for (int P = 0; P < 16; ++P) {
    const int j = P >> 2, v = P & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = src[tile_col(t, l, P, h)] & 15u;
#pragma unroll
      for (int b = 0; b < 4; ++b) pl[b] |= ((c >> b) & 1u) << ((plane_bit(j, 2 * v + h) + b) & 31);
    }
  }
  const uint64_t off = code_offset(s, t, l, n_kt, 4);
#pragma unroll
  for (int b = 0; b < 4; ++b)
    *reinterpret_cast<uint32_t *>(out + (uint64_t)(3 - b) * plane_bytes + off) = pl[b];
}

__global__ void __launch_bounds__(256)
pack_meta_kernel(const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int N,
                 int K, int G, uint16_t *__restrict__ s_out, uint8_t *__restrict__ z_out) {
  const int n_kt = K / kTileK, gpt = kTileK / G, ng = K / G;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)N * ng) return;
  const int n = (int)(id / ng), g = (int)(id % ng);
  const int s = n / kStripRows, r = n % kStripRows;
  const int t = g / gpt, gi = g % gpt;
  const uint64_t dst = meta_index(s, t, r, gi, n_kt, gpt);
  s_out[dst] = scales[id];
  z_out[dst] = zeros[id];
}

__global__ void __launch_bounds__(256)
pack_lut_kernel(const uint16_t *__restrict__ lut, int N, int K, int q, uint16_t *__restrict__ out) {
  const int n_kt = K / kTileK, nq = 1 << q;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)N * n_kt * nq) return;
  const int j = (int)(id % nq);
  const int t = (int)((id / nq) % n_kt);
  const int n = (int)(id / nq / n_kt);
  out[lut_index(n / kStripRows, t, n % kStripRows, j, n_kt, nq)] = lut[((int64_t)n * n_kt + t) * 16 + j];
}

// Debug read-back: one thread per (strip, tile, lane), same decode as the
// expert kernels.  INT: (c - 0) pairs; bit-plane: the q-bit indices.
template <int B>
__global__ void __launch_bounds__(256)
unpack_int_kernel(const uint8_t *__restrict__ packed, int N, int K, uint8_t *__restrict__ out) {
  const int n_kt = K / kTileK;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)(N / kStripRows) * n_kt * 64) return;
  const int l = (int)(id & 63);
  const int t = (int)((id >> 6) % n_kt);
  const int s = (int)((id >> 6) / n_kt);
  uint32_t d[B];
#pragma unroll
  for (int e = 0; e < B; ++e) d[e] = *reinterpret_cast<const uint32_t *>(packed + int_word_offset(s, t, l, e, n_kt, B));
  PairConst pc[9];
  fill_pair_consts<B>(pc, 0u);
  uint8_t *dst = out + (int64_t)(s * kStripRows + (l & 15)) * K;
#pragma unroll
  for (int P = 0; P < 16; ++P) {
    const f16x2 cz = as_h2(int_pair_cz<B>(d, P, pc));
    dst[tile_col(t, l, P, 0)] = (uint8_t)(int)(float)cz[0];
    dst[tile_col(t, l, P, 1)] = (uint8_t)(int)(float)cz[1];
  }
}

template <int Q>
__global__ void __launch_bounds__(256)
unpack_planes_kernel(const uint8_t *__restrict__ packed, uint64_t plane_bytes, int N, int K,
                     uint8_t *__restrict__ out) {
  const int n_kt = K / kTileK;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)(N / kStripRows) * n_kt * 64) return;
  const int l = (int)(id & 63);
  const int t = (int)((id >> 6) % n_kt);
  const int s = (int)((id >> 6) / n_kt);
  const uint64_t off = code_offset(s, t, l, n_kt, 4);
  uint32_t pl[Q];
#pragma unroll
  for (int u = 0; u < Q; ++u) pl[u] = *reinterpret_cast<const uint32_t *>(packed + u * plane_bytes + off);
  uint8_t *dst = out + (int64_t)(s * kStripRows + (l & 15)) * K;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dst[tile_col(t, l, 4 * j + i / 2, i % 2)] = (uint8_t)plane_index<Q>(pl, 4 * (i / 4) + j, i % 4);
  }
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  size_t total;
  size_t desc_off;
  std::vector<size_t> codes_off, scales_off, zeros_off, lut_off, U_off, V_off;
  std::vector<size_t> Us_off, Vs_off;
};

static void block_nk(const LayerDims &d, int blk, int *N, int *K) {
  if (blk < 2) { *N = d.I; *K = d.H; } else { *N = d.H; *K = d.I; }
}

static moeq_status validate(const moeq_layer_desc *d) {
  if (!d) return fail(MOEQ_ERR_INVALID, "pack: null description");
  if (d->E < 1 || d->E > 256) return fail(MOEQ_ERR_INVALID, "pack: E=%d not in 1..256", d->E);
  if (d->H <= 0 || d->I <= 0) return fail(MOEQ_ERR_INVALID, "pack: H=%d I=%d must be positive", d->H, d->I);
  if (d->H % kTileK || d->I % kTileK)
    return fail(MOEQ_ERR_UNSUPPORTED, "pack: H=%d and I=%d must be multiples of 128", d->H, d->I);
  if (d->fmt != MOEQ_FMT_INT && d->fmt != MOEQ_FMT_BITPLANE)
    return fail(MOEQ_ERR_INVALID, "pack: unknown format %d", d->fmt);
  if (d->fmt == MOEQ_FMT_INT && d->G != 64 && d->G != 128)
    return fail(MOEQ_ERR_UNSUPPORTED, "pack: INT group G=%d not in {64,128}", d->G);
  if (d->fmt == MOEQ_FMT_BITPLANE && d->G != 128)
    return fail(MOEQ_ERR_UNSUPPORTED, "pack: bit-plane group G=%d must be 128", d->G);
  if (!d->bits || !d->codes) return fail(MOEQ_ERR_INVALID, "pack: bits/codes arrays missing");
  const int nb = 3 * d->E;
  for (int b = 0; b < nb; ++b) {
    if (d->bits[b] < 2 || d->bits[b] > 4)
      return fail(MOEQ_ERR_INVALID, "pack: bits[%d]=%d not in {2,3,4}", b, d->bits[b]);
    if (!d->codes[b]) return fail(MOEQ_ERR_INVALID, "pack: codes[%d] is null", b);
    if (d->fmt == MOEQ_FMT_INT) {
      if (!d->scales || !d->zeros || !d->scales[b] || !d->zeros[b])
        return fail(MOEQ_ERR_INVALID, "pack: scales/zeros of block %d missing", b);
    } else if (!d->luts || !d->luts[b]) {
      return fail(MOEQ_ERR_INVALID, "pack: lut of block %d missing", b);
    }
  }
  if (d->r < 0 || d->r > 64 || d->r % 8)
    return fail(MOEQ_ERR_INVALID, "pack: r=%d must be a multiple of 8 in 0..64", d->r);
  if (d->r > 0) {
    if (!d->U || !d->V) return fail(MOEQ_ERR_INVALID, "pack: U/V arrays missing for r=%d", d->r);
    for (int b = 0; b < nb; ++b)
      if (!d->U[b] || !d->V[b]) return fail(MOEQ_ERR_INVALID, "pack: U/V of block %d missing", b);
  }
  if (d->rs < 0 || d->rs > 64 || d->rs % 8)
    return fail(MOEQ_ERR_INVALID, "pack: rs=%d must be a multiple of 8 in 0..64", d->rs);
  if (d->rs > 0) {
    if (d->share < 1 || d->share > d->E) return fail(MOEQ_ERR_INVALID, "pack: share=%d invalid", d->share);
    if (!d->Us || !d->Vs) return fail(MOEQ_ERR_INVALID, "pack: Us/Vs arrays missing for rs=%d", d->rs);
    const int ng = (d->E + d->share - 1) / d->share;
    for (int b = 0; b < 3 * ng; ++b)
      if (!d->Us[b] || !d->Vs[b]) return fail(MOEQ_ERR_INVALID, "pack: Us/Vs of group block %d missing", b);
  }
  return MOEQ_OK;
}

static Plan make_plan(const moeq_layer_desc *d) {
  LayerDims dims{d->E, d->H, d->I, d->G, d->fmt, d->r, d->rs, d->share};
  Plan p;
  const int nb = 3 * d->E;
  size_t off = 0;
  p.desc_off = off;
  off = align256(off + sizeof(BlockDesc) * nb);
  p.codes_off.resize(nb); p.scales_off.resize(nb, 0); p.zeros_off.resize(nb, 0);
  p.lut_off.resize(nb, 0); p.U_off.resize(nb, 0); p.V_off.resize(nb, 0);
  for (int b = 0; b < nb; ++b) {
    int N, K;
    block_nk(dims, b % 3, &N, &K);
    const size_t nk = (size_t)N * K;
    const int bits = d->bits[b];
    p.codes_off[b] = off;
    if (d->fmt == MOEQ_FMT_INT) {
      off = align256(off + nk * bits / 8);
      p.scales_off[b] = off;
      off = align256(off + (nk / d->G) * 2);
      p.zeros_off[b] = off;
      off = align256(off + nk / d->G);
    } else {
      off = align256(off + 4 * align256(nk / 8));
      p.lut_off[b] = off;
      // room for a 16-entry table per (row, tile): a later commit to any q
      // rewrites the table in place
      off = align256(off + (nk / kTileK) * 32);
    }
    if (d->r > 0) {
      p.U_off[b] = off; off = align256(off + (size_t)N * d->r * 2);
      p.V_off[b] = off; off = align256(off + (size_t)d->r * K * 2);
    }
  }
  if (d->rs > 0) {
    const int ng = (d->E + d->share - 1) / d->share;
    p.Us_off.resize(3 * ng); p.Vs_off.resize(3 * ng);
    for (int b = 0; b < 3 * ng; ++b) {
      int N, K;
      block_nk(dims, b % 3, &N, &K);
      p.Us_off[b] = off; off = align256(off + (size_t)N * d->rs * 2);
      p.Vs_off[b] = off; off = align256(off + (size_t)d->rs * K * 2);
    }
  }
  p.total = off;
  return p;
}

static inline unsigned nblocks(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace moeq

using namespace moeq;

MOEQ_API moeq_status moeq_pack_size(const moeq_layer_desc *d, size_t *device_bytes) {
  moeq_status st = validate(d);
  if (st != MOEQ_OK) return st;
  if (!device_bytes) return fail(MOEQ_ERR_INVALID, "pack_size: null output");
  *device_bytes = make_plan(d).total;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_pack(const moeq_layer_desc *d, void *device_buf, size_t bytes,
                               hipStream_t stream, moeq_layer **out) {
  moeq_status st = validate(d);
  if (st != MOEQ_OK) return st;
  if (!device_buf || !out) return fail(MOEQ_ERR_INVALID, "pack: null buffer or output handle");
  if (reinterpret_cast<uintptr_t>(device_buf) & 255)
    return fail(MOEQ_ERR_INVALID, "pack: device buffer must be 256-byte aligned");
  const Plan p = make_plan(d);
  if (bytes < p.total) return fail(MOEQ_ERR_WORKSPACE, "pack: buffer has %zu bytes, needs %zu", bytes, p.total);

  moeq_layer *L = new (std::nothrow) moeq_layer();
  if (!L) return fail(MOEQ_ERR_INVALID, "pack: out of host memory");
  L->dims = LayerDims{d->E, d->H, d->I, d->G, d->fmt, d->r, d->rs, d->share};
  L->buf = static_cast<uint8_t *>(device_buf);
  L->bytes = bytes;
  L->d_desc = reinterpret_cast<BlockDesc *>(L->buf + p.desc_off);
  const int nb = 3 * d->E;
  L->bits.assign(d->bits, d->bits + nb);
  L->h_desc.resize(nb);
  L->block_alg_bytes.resize(nb);
  const int ngrp = d->rs > 0 ? (d->E + d->share - 1) / d->share : 0;
  L->shared_alg_bytes.assign(3 * ngrp, 0);

  for (int b = 0; b < nb; ++b) {
    int N, K;
    block_nk(L->dims, b % 3, &N, &K);
    const int bits = d->bits[b];
    const int n_kt = K / kTileK;
    const int64_t lanes = (int64_t)(N / kStripRows) * n_kt * 64;
    BlockDesc &bd = L->h_desc[b];
    std::memset(&bd, 0, sizeof(bd));
    bd.N = N; bd.K = K; bd.bits = bits; bd.fmt = d->fmt;
    bd.codes = L->buf + p.codes_off[b];
    uint8_t *codes_dst = L->buf + p.codes_off[b];
    size_t alg = 0;
    const size_t nk = (size_t)N * K;
    if (d->fmt == MOEQ_FMT_INT) {
      bd.scales = reinterpret_cast<const uint16_t *>(L->buf + p.scales_off[b]);
      bd.zeros = L->buf + p.zeros_off[b];
      switch (bits) {
        case 2: hipLaunchKernelGGL(pack_int_kernel<2>, dim3(nblocks(lanes)), dim3(256), 0, stream, d->codes[b], N, K, codes_dst); break;
        case 3: hipLaunchKernelGGL(pack_int_kernel<3>, dim3(nblocks(lanes)), dim3(256), 0, stream, d->codes[b], N, K, codes_dst); break;
        default: hipLaunchKernelGGL(pack_int_kernel<4>, dim3(nblocks(lanes)), dim3(256), 0, stream, d->codes[b], N, K, codes_dst); break;
      }
      hipLaunchKernelGGL(pack_meta_kernel, dim3(nblocks((int64_t)nk / d->G)), dim3(256), 0, stream,
                         d->scales[b], d->zeros[b], N, K, d->G,
                         reinterpret_cast<uint16_t *>(L->buf + p.scales_off[b]), L->buf + p.zeros_off[b]);
      alg = nk * bits / 8 + (nk / d->G) * 3;
    } else {
      bd.plane_bytes = align256(nk / 8);
      bd.lut = reinterpret_cast<const uint16_t *>(L->buf + p.lut_off[b]);
      hipLaunchKernelGGL(pack_planes_kernel, dim3(nblocks(lanes)), dim3(256), 0, stream,
                         d->codes[b], N, K, codes_dst, (uint64_t)bd.plane_bytes);
      hipLaunchKernelGGL(pack_lut_kernel, dim3(nblocks((int64_t)N * n_kt << bits)), dim3(256), 0, stream,
                         d->luts[b], N, K, bits, reinterpret_cast<uint16_t *>(L->buf + p.lut_off[b]));
      alg = nk * bits / 8 + (nk / kTileK) * ((size_t)2 << bits);
    }
    if (d->r > 0) {
      bd.U = reinterpret_cast<const uint16_t *>(L->buf + p.U_off[b]);
      bd.V = reinterpret_cast<const uint16_t *>(L->buf + p.V_off[b]);
      if (hipMemcpyAsync(L->buf + p.U_off[b], d->U[b], (size_t)N * d->r * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess ||
          hipMemcpyAsync(L->buf + p.V_off[b], d->V[b], (size_t)d->r * K * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess) {
        delete L;
        return fail(MOEQ_ERR_HIP, "pack: factor copy failed: %s", hipGetErrorString(hipGetLastError()));
      }
      alg += (size_t)(N + K) * d->r * 2;
    }
    L->block_alg_bytes[b] = alg;
  }
  for (int gb = 0; gb < 3 * ngrp; ++gb) {
    int N, K;
    block_nk(L->dims, gb % 3, &N, &K);
    if (hipMemcpyAsync(L->buf + p.Us_off[gb], d->Us[gb], (size_t)N * d->rs * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess ||
        hipMemcpyAsync(L->buf + p.Vs_off[gb], d->Vs[gb], (size_t)d->rs * K * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess) {
      delete L;
      return fail(MOEQ_ERR_HIP, "pack: shared factor copy failed: %s", hipGetErrorString(hipGetLastError()));
    }
    L->shared_alg_bytes[gb] = (size_t)(N + K) * d->rs * 2;
  }
  if (ngrp > 0) {
    for (int b = 0; b < nb; ++b) {
      const int gb = (b / 3 / d->share) * 3 + b % 3;
      L->h_desc[b].Us = reinterpret_cast<const uint16_t *>(L->buf + p.Us_off[gb]);
      L->h_desc[b].Vs = reinterpret_cast<const uint16_t *>(L->buf + p.Vs_off[gb]);
    }
  }
  moeq_status ls = check_launch("pack");
  if (ls != MOEQ_OK) { delete L; return ls; }
  if (hipMemcpyAsync(L->d_desc, L->h_desc.data(), sizeof(BlockDesc) * nb, hipMemcpyHostToDevice, stream) != hipSuccess) {
    delete L;
    return fail(MOEQ_ERR_HIP, "pack: descriptor copy failed: %s", hipGetErrorString(hipGetLastError()));
  }
  L->resident.assign(nb, d->fmt == MOEQ_FMT_BITPLANE ? 4 : 0);
  L->desired.assign(d->bits, d->bits + nb);
  L->reload_pending.assign(nb, 0);
  if (d->fmt == MOEQ_FMT_BITPLANE) {
    L->commit_ev.reserve(nb);
    L->copy_ev.reserve(nb);
    for (int b = 0; b < nb; ++b) {
      hipEvent_t e0, e1;
      if (hipEventCreateWithFlags(&e0, hipEventDisableTiming) != hipSuccess) { delete L; return fail(MOEQ_ERR_HIP, "pack: event creation failed"); }
      L->commit_ev.push_back(e0);
      if (hipEventCreateWithFlags(&e1, hipEventDisableTiming) != hipSuccess) { delete L; return fail(MOEQ_ERR_HIP, "pack: event creation failed"); }
      L->copy_ev.push_back(e1);
    }
  }
  *out = L;
  return MOEQ_OK;
}

MOEQ_API void moeq_layer_destroy(moeq_layer *L) { delete L; }

MOEQ_API moeq_status moeq_layer_block_bytes(const moeq_layer *L, int32_t e, int32_t blk, size_t *bytes) {
  if (!L || !bytes) return fail(MOEQ_ERR_INVALID, "layer_block_bytes: null argument");
  if (e < 0 || e >= L->dims.E || blk < 0 || blk > 2) return fail(MOEQ_ERR_INVALID, "layer_block_bytes: bad block (%d,%d)", e, blk);
  *bytes = L->block_alg_bytes[3 * e + blk];
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_layer_shared_bytes(const moeq_layer *L, int32_t group, int32_t blk, size_t *bytes) {
  if (!L || !bytes) return fail(MOEQ_ERR_INVALID, "layer_shared_bytes: null argument");
  const int ng = (int)L->shared_alg_bytes.size() / 3;
  if (group < 0 || group >= ng || blk < 0 || blk > 2) {
    *bytes = 0;
    if (ng == 0) return MOEQ_OK;
    return fail(MOEQ_ERR_INVALID, "layer_shared_bytes: bad group block (%d,%d)", group, blk);
  }
  *bytes = L->shared_alg_bytes[3 * group + blk];
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_debug_unpack(const moeq_layer *L, int32_t e, int32_t blk, uint8_t *out,
                                       hipStream_t stream) {
  if (!L || !out) return fail(MOEQ_ERR_INVALID, "debug_unpack: null argument");
  if (e < 0 || e >= L->dims.E || blk < 0 || blk > 2) return fail(MOEQ_ERR_INVALID, "debug_unpack: bad block (%d,%d)", e, blk);
  const BlockDesc &bd = L->h_desc[3 * e + blk];
  const int64_t lanes = (int64_t)(bd.N / kStripRows) * (bd.K / kTileK) * 64;
  prof_begin("debug_unpack", stream);
  if (bd.fmt == MOEQ_FMT_INT) {
    switch (bd.bits) {
      case 2: hipLaunchKernelGGL(unpack_int_kernel<2>, dim3(nblocks(lanes)), dim3(256), 0, stream, bd.codes, bd.N, bd.K, out); break;
      case 3: hipLaunchKernelGGL(unpack_int_kernel<3>, dim3(nblocks(lanes)), dim3(256), 0, stream, bd.codes, bd.N, bd.K, out); break;
      default: hipLaunchKernelGGL(unpack_int_kernel<4>, dim3(nblocks(lanes)), dim3(256), 0, stream, bd.codes, bd.N, bd.K, out); break;
    }
  } else {
    switch (bd.bits) {
      case 2: hipLaunchKernelGGL(unpack_planes_kernel<2>, dim3(nblocks(lanes)), dim3(256), 0, stream, bd.codes, (uint64_t)bd.plane_bytes, bd.N, bd.K, out); break;
      case 3: hipLaunchKernelGGL(unpack_planes_kernel<3>, dim3(nblocks(lanes)), dim3(256), 0, stream, bd.codes, (uint64_t)bd.plane_bytes, bd.N, bd.K, out); break;
      default: hipLaunchKernelGGL(unpack_planes_kernel<4>, dim3(nblocks(lanes)), dim3(256), 0, stream, bd.codes, (uint64_t)bd.plane_bytes, bd.N, bd.K, out); break;
    }
  }
  prof_end("debug_unpack", stream);
  return check_launch("debug_unpack");
}

namespace moeq {

// Stream-ordered update of one block's committed bit-plane count.
__global__ void set_bits_kernel(BlockDesc *d, int32_t bits) { d->bits = bits; }

}  // namespace moeq

MOEQ_API moeq_status moeq_commit_bits(moeq_layer *L, int32_t e, int32_t blk, int32_t q, const uint16_t *lut,
                                      hipStream_t stream) {
  if (!L) return fail(MOEQ_ERR_INVALID, "commit_bits: null layer");
  if (e < 0 || e >= L->dims.E || blk < 0 || blk > 2) return fail(MOEQ_ERR_INVALID, "commit_bits: bad block (%d,%d)", e, blk);
  if (L->dims.fmt != MOEQ_FMT_BITPLANE)
    return fail(MOEQ_ERR_UNSUPPORTED, "commit_bits: only bit-plane layers change bitwidth after packing");
  if (q < 2 || q > 4) return fail(MOEQ_ERR_INVALID, "commit_bits: q=%d not in {2,3,4}", q);
  if (!lut) return fail(MOEQ_ERR_INVALID, "commit_bits: null LUT");
  const int b = 3 * e + blk;
  if (q > L->resident[b])
    return fail(MOEQ_ERR_INVALID, "commit_bits: q=%d needs planes %d..%d of block (%d,%d), which are released "
                "(reload them with moeq_plane_reload first)", q, L->resident[b], q - 1, e, blk);
  BlockDesc &bd = L->h_desc[b];
  const int n_kt = bd.K / kTileK;
  // a reload of this block's planes lands before the new bitwidth is used
  if (L->reload_pending[b]) {
    if (hipStreamWaitEvent(stream, L->copy_ev[b], 0) != hipSuccess)
      return fail(MOEQ_ERR_HIP, "commit_bits: stream wait failed: %s", hipGetErrorString(hipGetLastError()));
    L->reload_pending[b] = 0;
  }
  prof_begin("commit_bits", stream);
  hipLaunchKernelGGL(pack_lut_kernel, dim3(nblocks((int64_t)bd.N * n_kt << q)), dim3(256), 0, stream,
                     lut, bd.N, bd.K, q, const_cast<uint16_t *>(bd.lut));
  hipLaunchKernelGGL(set_bits_kernel, dim3(1), dim3(1), 0, stream, L->d_desc + b, q);
  prof_end("commit_bits", stream);
  moeq_status st = check_launch("commit_bits");
  if (st != MOEQ_OK) return st;
  // releases of this block wait for everything enqueued up to here
  if (hipEventRecord(L->commit_ev[b], stream) != hipSuccess)
    return fail(MOEQ_ERR_HIP, "commit_bits: event record failed: %s", hipGetErrorString(hipGetLastError()));
  const size_t nk = (size_t)bd.N * bd.K;
  const size_t old_codes = nk * bd.bits / 8 + (nk / kTileK) * ((size_t)2 << bd.bits);
  const size_t new_codes = nk * q / 8 + (nk / kTileK) * ((size_t)2 << q);
  L->block_alg_bytes[b] = L->block_alg_bytes[b] - old_codes + new_codes;
  bd.bits = q;
  L->bits[b] = (uint8_t)q;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_committed_bits(const moeq_layer *L, int32_t e, int32_t blk, int32_t *q) {
  if (!L || !q) return fail(MOEQ_ERR_INVALID, "committed_bits: null argument");
  if (e < 0 || e >= L->dims.E || blk < 0 || blk > 2) return fail(MOEQ_ERR_INVALID, "committed_bits: bad block (%d,%d)", e, blk);
  *q = L->h_desc[3 * e + blk].bits;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_plane_region(const moeq_layer *L, int32_t e, int32_t blk, int32_t plane, void **ptr,
                                       size_t *bytes) {
  if (!L || !ptr || !bytes) return fail(MOEQ_ERR_INVALID, "plane_region: null argument");
  if (e < 0 || e >= L->dims.E || blk < 0 || blk > 2) return fail(MOEQ_ERR_INVALID, "plane_region: bad block (%d,%d)", e, blk);
  if (L->dims.fmt != MOEQ_FMT_BITPLANE) return fail(MOEQ_ERR_UNSUPPORTED, "plane_region: not a bit-plane layer");
  if (plane < 0 || plane > 3) return fail(MOEQ_ERR_INVALID, "plane_region: plane=%d not in 0..3", plane);
  const BlockDesc &bd = L->h_desc[3 * e + blk];
  *ptr = const_cast<uint8_t *>(bd.codes) + (size_t)plane * bd.plane_bytes;
  *bytes = bd.plane_bytes;
  return MOEQ_OK;
}

// ---- page movement ([PW] "What carries the argument" and Figure 4: a
// lowered bitwidth is committed before its pages are released; released
// pages come back before a higher bitwidth is committed).

static moeq_status plane_block(const moeq_layer *L, int32_t e, int32_t blk, const char *what, int *b) {
  if (!L) return fail(MOEQ_ERR_INVALID, "%s: null layer", what);
  if (e < 0 || e >= L->dims.E || blk < 0 || blk > 2) return fail(MOEQ_ERR_INVALID, "%s: bad block (%d,%d)", what, e, blk);
  if (L->dims.fmt != MOEQ_FMT_BITPLANE) return fail(MOEQ_ERR_UNSUPPORTED, "%s: not a bit-plane layer", what);
  *b = 3 * e + blk;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_resident_planes(const moeq_layer *L, int32_t e, int32_t blk, int32_t *n) {
  int b;
  moeq_status st = plane_block(L, e, blk, "resident_planes", &b);
  if (st != MOEQ_OK) return st;
  if (!n) return fail(MOEQ_ERR_INVALID, "resident_planes: null output");
  *n = L->resident[b];
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_set_desired_bits(moeq_layer *L, int32_t e, int32_t blk, int32_t d) {
  int b;
  moeq_status st = plane_block(L, e, blk, "set_desired_bits", &b);
  if (st != MOEQ_OK) return st;
  if (d < 2 || d > 4) return fail(MOEQ_ERR_INVALID, "set_desired_bits: d=%d not in {2,3,4}", d);
  L->desired[b] = (uint8_t)d;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_desired_bits(const moeq_layer *L, int32_t e, int32_t blk, int32_t *d) {
  int b;
  moeq_status st = plane_block(L, e, blk, "desired_bits", &b);
  if (st != MOEQ_OK) return st;
  if (!d) return fail(MOEQ_ERR_INVALID, "desired_bits: null output");
  *d = L->desired[b];
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_plane_release(moeq_layer *L, int32_t e, int32_t blk, void *host, size_t host_bytes,
                                        hipStream_t stream) {
  int b;
  moeq_status st = plane_block(L, e, blk, "plane_release", &b);
  if (st != MOEQ_OK) return st;
  const BlockDesc &bd = L->h_desc[b];
  const int q = bd.bits, res = L->resident[b];
  if (q >= res) return MOEQ_OK;                        // nothing above the committed bitwidth
  const size_t pb = bd.plane_bytes;
  if (!host) return fail(MOEQ_ERR_INVALID, "plane_release: null host buffer");
  if (host_bytes < (size_t)res * pb)
    return fail(MOEQ_ERR_INVALID, "plane_release: host buffer has %zu bytes, planes up to %d need %zu", host_bytes,
                res - 1, (size_t)res * pb);
  // after every kernel enqueued before the block's last commit
  if (hipStreamWaitEvent(stream, L->commit_ev[b], 0) != hipSuccess ||
      hipMemcpyAsync(static_cast<uint8_t *>(host) + (size_t)q * pb, bd.codes + (size_t)q * pb, (size_t)(res - q) * pb,
                     hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipEventRecord(L->copy_ev[b], stream) != hipSuccess)
    return fail(MOEQ_ERR_HIP, "plane_release: %s", hipGetErrorString(hipGetLastError()));
  L->resident[b] = (uint8_t)q;
  L->reload_pending[b] = 0;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_plane_reload(moeq_layer *L, int32_t e, int32_t blk, int32_t q, const void *host,
                                       size_t host_bytes, hipStream_t stream) {
  int b;
  moeq_status st = plane_block(L, e, blk, "plane_reload", &b);
  if (st != MOEQ_OK) return st;
  if (q < 2 || q > 4) return fail(MOEQ_ERR_INVALID, "plane_reload: q=%d not in {2,3,4}", q);
  const int res = L->resident[b];
  if (q <= res) return MOEQ_OK;                         // already resident
  const BlockDesc &bd = L->h_desc[b];
  const size_t pb = bd.plane_bytes;
  if (!host) return fail(MOEQ_ERR_INVALID, "plane_reload: null host buffer");
  if (host_bytes < (size_t)q * pb)
    return fail(MOEQ_ERR_INVALID, "plane_reload: host buffer has %zu bytes, planes up to %d need %zu", host_bytes, q - 1,
                (size_t)q * pb);
  if (hipMemcpyAsync(const_cast<uint8_t *>(bd.codes) + (size_t)res * pb,
                     static_cast<const uint8_t *>(host) + (size_t)res * pb, (size_t)(q - res) * pb,
                     hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(L->copy_ev[b], stream) != hipSuccess)
    return fail(MOEQ_ERR_HIP, "plane_reload: %s", hipGetErrorString(hipGetLastError()));
  L->resident[b] = (uint8_t)q;
  L->reload_pending[b] = 1;
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_plane_event(const moeq_layer *L, int32_t e, int32_t blk, hipEvent_t *ev) {
  int b;
  moeq_status st = plane_block(L, e, blk, "plane_event", &b);
  if (st != MOEQ_OK) return st;
  if (!ev) return fail(MOEQ_ERR_INVALID, "plane_event: null output");
  *ev = L->copy_ev[b];
  return MOEQ_OK;
}
