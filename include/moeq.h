/*
 * moeq.h — C ABI of libmoeq: a routed Mixture-of-Experts expert layer on
 * low-bit group-quantized weights with low-rank compensators, for AMD
 * Instinct MI355X (gfx950).
 *
 *   y_t = sum_{j<k} g_{t,j} * Down_e( SiLU(Gate_e x_t) * Up_e x_t ),  e = ids[t][j]
 *   every linear L(v) = W_hat v + [comp] * ( U (V v) + U_G (V_G v) )
 *
 * Sources (the pages this library follows; each entry point below names the
 * passage that defines its operation):
 *   [MiLo]   "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
 *            Compensators", abstract — under-4-bit MoE weights plus low-rank
 *            compensators.
 *   [PW]     "PagedWeight: Efficient MoE LLM Serving with Dynamic Quality-Aware
 *            Weight Quantization" (review page) — "What carries the argument"
 *            (weight pages, committed bitwidth per expert linear block),
 *            Figure 3 caption (bit-plane format with a per-tensor LUT of
 *            bitwidth-specific centroids), referee summary (a fused
 *            mixed-precision MoE kernel that executes variable bitwidths).
 *   [TileQ]  "TileQ: Efficient Low-Rank Quantization of Mixture-of-Experts
 *            with 2D Tiling", abstract — low-rank factors shared across
 *            experts; several low-rank expert computations fused in one pass.
 *   [BEAM]   "Bandwidth-Efficient Adaptive Mixture-of-Experts via Low-Rank
 *            Compensation", abstract — compensation only for each token's
 *            top-n (n < k) experts.
 *   [MxMoE]  "MxMoE: Mixed-precision Quantization for MoE with Accuracy and
 *            Performance Co-Design", abstract — per-linear-block bitwidths;
 *            uneven expert activation frequencies.
 *
 * Conventions for every entry point:
 *   - Pointers marked DEVICE are device memory owned by the caller (the
 *     library never allocates device memory); pointers marked HOST are read
 *     during the call only.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     validation error nothing is written, and the call returns
 *     MOEQ_ERR_INVALID (bad argument), MOEQ_ERR_UNSUPPORTED (valid but not
 *     implemented) or MOEQ_ERR_WORKSPACE (workspace too small);
 *     moeq_last_error() returns a thread-local description.
 *   - Work is enqueued asynchronously on the given stream; there are no host
 *     synchronisations or device-to-host reads.  A failed kernel launch
 *     returns MOEQ_ERR_HIP; device faults surface at the caller's next
 *     synchronisation.
 *   - Identical inputs give bit-identical outputs (no atomics on any output).
 *   - A packed layer may be used from several streams at once if every call
 *     has its own workspace and outputs.
 *   - Matrices are row-major.  fp16 values are passed as uint16_t bit
 *     patterns.  A block is one linear of one expert, numbered
 *     e * 3 + blk with blk 0 = gate [I, H], 1 = up [I, H], 2 = down [H, I]
 *     (rows = outputs N, columns = inputs K).
 *   - No C++ exception crosses this boundary.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOEQ_OK = 0,
  MOEQ_ERR_INVALID = 1,
  MOEQ_ERR_UNSUPPORTED = 2,
  MOEQ_ERR_WORKSPACE = 3,
  MOEQ_ERR_HIP = 4
} moeq_status;

typedef enum { MOEQ_FMT_INT = 0, MOEQ_FMT_BITPLANE = 1 } moeq_format;
typedef enum { MOEQ_F16 = 0, MOEQ_F32 = 1 } moeq_dtype;

/* Name of a status code (static string). */
const char *moeq_status_string(moeq_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char *moeq_last_error(void);
/* ABI version of this library (increments on incompatible changes). */
int32_t moeq_abi_version(void);

/* ------------------------------------------------------------ encoding -- */

/*
 * moeq_quantize_rtn — asymmetric round-to-nearest group quantization of one
 * fp16 block ([MiLo] under-4-bit expert weights; [MxMoE] per-block bitwidth).
 * For every row n and group g of G consecutive columns, in float64:
 *   lo = min(0, min w), hi = max(0, max w)
 *   s16 = fp16((hi - lo) / (2^bits - 1)) rounded once half-to-even,
 *         and s16 = 1 when hi == lo or the rounded value is 0
 *   z = clamp(rint(-lo / s16), 0, 2^bits - 1)
 *   c = clamp(rint(w / s16) + z, 0, 2^bits - 1),  rint = half to even.
 *   w      DEVICE [N, K] fp16 (finite)
 *   codes  DEVICE [N, K] uint8 out, one code per byte
 *   scales DEVICE [N, K/G] fp16 out;  zeros DEVICE [N, K/G] uint8 out
 *   N, K > 0; G in {64, 128} dividing K (any G >= 2 dividing K is accepted);
 *   bits in {2, 3, 4}.
 */
moeq_status moeq_quantize_rtn(const uint16_t *w, int32_t N, int32_t K, int32_t G,
                              int32_t bits, uint8_t *codes, uint16_t *scales,
                              uint8_t *zeros, hipStream_t stream);

/*
 * moeq_build_lut — per-(row, group) lookup table of a block committed to q
 * bit-planes ([PW] Figure 3 caption: subsets of bit-planes give the
 * effective bitwidth; the LUT holds bitwidth-specific centroid values).
 * Parent codes are the 4-bit RTN codes of the block (moeq_quantize_rtn with
 * bits = 4); the q-bit index of a weight is code >> (4 - q).  Slot j < 2^q is
 * fp16 of the float64 mean of the group's fp16 weights with index j; an empty
 * slot gets fp16(s16 * (j * 2^(4-q) + (2^(4-q) - 1) / 2 - z)); slots
 * j >= 2^q are 0.
 *   w DEVICE [N, K] fp16; codes4 DEVICE [N, K] uint8 (< 16);
 *   scales / zeros DEVICE [N, K/G] (from the same 4-bit quantization);
 *   lut DEVICE [N, K/G, 16] fp16 out;  q in {2, 3, 4}; G divides K, G <= 256.
 */
moeq_status moeq_build_lut(const uint16_t *w, const uint8_t *codes4,
                           const uint16_t *scales, const uint8_t *zeros, int32_t N,
                           int32_t K, int32_t G, int32_t q, uint16_t *lut,
                           hipStream_t stream);

/*
 * moeq_fit_lowrank — rank-r compensator factors of the quantization residual
 * (data preparation, before the path; [MiLo] abstract: low-rank
 * compensators of the quantized experts; [TileQ] abstract: factors shared
 * by a group of experts).  The residual is the mean over n_mat blocks
 *   R = (1/n_mat) sum_m (w_m - s_m * (c_m - z_m))
 * (n_mat = 1: one block's compensator; n_mat > 1: the pair shared by a
 * group, which minimizes sum_m ||R_m - U V||_F).  U V approximates the
 * rank-r truncation of R by randomized subspace iteration (Halko,
 * Martinsson and Tropp): Y = R omega, power_iters steps of Y = R orth(R^T
 * orth(Y)), Q = orth(Y), then the exact SVD of Q^T R; the singular values
 * are split evenly: U = P sqrt(S), V = sqrt(S) Q'^T.
 *   w DEVICE [n_mat, N, K] fp16; codes DEVICE [n_mat, N, K] uint8;
 *   scales DEVICE [n_mat, N, K/G] fp16; zeros DEVICE [n_mat, N, K/G] uint8
 *   (the RTN outputs of moeq_quantize_rtn for each block);
 *   omega DEVICE [K, l] fp32, drawn by the caller (e.g. N(0, 1));
 *   1 <= r <= l <= min(N, K, 128); power_iters in 0..16;
 *   U DEVICE [N, r] fp16 out; V DEVICE [r, K] fp16 out;
 *   ws DEVICE, at least moeq_fit_lowrank_workspace_size bytes.
 * The l x l factorizations run on the host in fp64: the call synchronizes
 * the stream (offline preparation, not part of the hot path).
 */
moeq_status moeq_fit_lowrank_workspace_size(int32_t N, int32_t K, int32_t r, int32_t l, size_t *bytes);
moeq_status moeq_fit_lowrank(const uint16_t *w, const uint8_t *codes, const uint16_t *scales,
                             const uint8_t *zeros, int32_t n_mat, int32_t N, int32_t K, int32_t G,
                             const float *omega, int32_t l, int32_t r, int32_t power_iters, uint16_t *U,
                             uint16_t *V, void *ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------- packed layer -- */

typedef struct moeq_layer moeq_layer; /* opaque host handle */

/*
 * Description of a quantized layer, read by moeq_pack only.  The pointer
 * arrays are HOST arrays (indexed by block e*3+blk, or group*3+blk for the
 * shared factors) of DEVICE pointers.
 *   E experts (1..256), H hidden, I intermediate; H and I multiples of 128.
 *   G quantization group along K: 64 or 128 for MOEQ_FMT_INT, 128 for
 *     MOEQ_FMT_BITPLANE.
 *   bits   HOST [E*3]: INT bitwidth b, or committed bit-plane count q; in {2,3,4}.
 *   codes  [E*3] -> [N*K] uint8: INT codes < 2^b, or 4-bit parent codes.
 *   scales, zeros [E*3] -> [N*(K/G)]  (MOEQ_FMT_INT only; NULL otherwise).
 *   luts   [E*3] -> [N*(K/G)*16] fp16 (MOEQ_FMT_BITPLANE only).
 *   r      per-expert compensator rank (0..64); U [E*3] -> [N*r], V -> [r*K].
 *   rs     shared compensator rank (0..64), share = experts per group
 *          (expert e uses group e / share); Us [(ceil(E/share))*3] -> [N*rs],
 *          Vs -> [rs*K] ([TileQ] factors shared across experts).
 */
typedef struct {
  int32_t E, H, I, G;
  int32_t fmt;
  const uint8_t *bits;
  const uint8_t *const *codes;
  const uint16_t *const *scales;
  const uint8_t *const *zeros;
  const uint16_t *const *luts;
  int32_t r;
  const uint16_t *const *U;
  const uint16_t *const *V;
  int32_t rs, share;
  const uint16_t *const *Us;
  const uint16_t *const *Vs;
} moeq_layer_desc;

/* Device bytes needed by moeq_pack for this description (validates it). */
moeq_status moeq_pack_size(const moeq_layer_desc *d, size_t *device_bytes);

/*
 * moeq_pack — lays the layer out for the expert kernels in caller-owned
 * device memory: codes in 16-row x 128-column tiles arranged for 128-bit
 * lane loads ([PW] weight pages: one region per expert linear block, the
 * bit-planes of a block stored plane by plane so that its top q planes are
 * contiguous), scales/zeros or LUTs beside them, fp16 factors, and a block
 * descriptor table.  The inputs may be freed once the stream has passed the
 * pack.  *out receives a host handle that owns no device memory; the caller
 * frees device_buf after moeq_layer_destroy and after all users finished.
 */
moeq_status moeq_pack(const moeq_layer_desc *d, void *device_buf, size_t bytes,
                      hipStream_t stream, moeq_layer **out);
void moeq_layer_destroy(moeq_layer *L);

/*
 * Algorithmic bytes of block (e, blk) as stored for the kernels: codes at b
 * bits per weight (top q planes for the bit-plane form), 2 B scale + 1 B
 * zero per (row, group) or 2^q * 2 B of LUT per (row, group), and the fp16
 * per-expert factors.  Shared factors are reported per group by
 * moeq_layer_shared_bytes.
 */
moeq_status moeq_layer_block_bytes(const moeq_layer *L, int32_t e, int32_t blk,
                                   size_t *bytes);
moeq_status moeq_layer_shared_bytes(const moeq_layer *L, int32_t group, int32_t blk,
                                    size_t *bytes);

/*
 * moeq_debug_unpack — reads block (e, blk) back from the packed layout with
 * the same in-register decode the expert kernels use, and writes one byte
 * per weight: the INT code, or the q-bit bit-plane index.  out DEVICE [N*K].
 */
moeq_status moeq_debug_unpack(const moeq_layer *L, int32_t e, int32_t blk,
                              uint8_t *out, hipStream_t stream);

/*
 * Runtime bitwidth of bit-plane blocks ([PW] "What carries the argument":
 * each expert linear block is a weight page of bit-planes plus the lookup
 * table of its committed bitwidth q; a page's bitwidth is lowered or
 * restored at run time and a change takes effect only once committed).
 *
 * moeq_commit_bits — make q the committed bit-plane count of block (e, blk)
 * for every call enqueued on `stream` after this one: the block's table is
 * rewritten from `lut` and its descriptor updated, both on `stream` (calls
 * already enqueued read the previous state; callers using several streams
 * order them themselves).  From then on the kernels read planes 0 .. q-1
 * (plane 0 = most significant) and the q-bit table.
 *   lut DEVICE [N][K/G][16] fp16, slots [0, 2^q) used (as from
 *   moeq_build_lut with this q); read during the call's stream work.
 *   Bit-plane layers only (MOEQ_ERR_UNSUPPORTED for INT); q in {2,3,4}.
 *   moeq_layer_block_bytes reports the new committed bytes afterwards.
 *
 * moeq_committed_bits — the committed q of a block (host-side state).
 *
 * moeq_plane_region — where plane `plane` (0 = most significant) of a
 * bit-plane block lives inside the packed buffer, and its size, so that a
 * caller can page a plane out (copy to host, reuse the bytes) while no
 * committed q reads it, and copy it back before committing a q that does.
 */
moeq_status moeq_commit_bits(moeq_layer *L, int32_t expert, int32_t block, int32_t q,
                             const uint16_t *lut, hipStream_t stream);

/*
 * Page movement of bit-plane blocks ([PW] "What carries the argument" and
 * the Figure 4 caption: at the offload threshold the lowered bitwidth is
 * committed and the pages above it are released to host memory; at the
 * reload threshold the pages come back before the higher bitwidth is
 * committed).  Every block keeps, host side, its committed q, the number of
 * its planes resident in device memory (4 after packing; planes are
 * released from the least significant one down) and a desired bitwidth d
 * (set by the caller's policy, e.g. from moeq_plan_reductions; d starts at
 * the packed q).  Nothing here allocates memory or synchronises the host.
 *
 * moeq_plane_release — copy the block's planes above its committed q to
 * host memory and mark them released.  The copy is enqueued on `stream`
 * after all work enqueued before the block's last moeq_commit_bits (the
 * kernels that may still read those planes).  Once the copy has completed
 * (work enqueued later on `stream`, or anything waiting on the event of
 * moeq_plane_event), the caller may reuse the released device bytes
 * (moeq_plane_region) until it reloads them.  A block with no plane above
 * its committed q is left as it is.
 *   host HOST [host_bytes], pinned, caller-owned; plane p is written at
 *   offset p * plane_bytes, for planes q .. resident - 1; host_bytes must
 *   cover the planes up to resident - 1.
 *
 * moeq_plane_reload — copy planes resident .. q-1 of the block back from
 * host memory (same layout) on `stream` and mark planes 0 .. q-1 resident.
 * The caller must have stopped using the reused bytes before the copy (in
 * `stream` order).  The next moeq_commit_bits of the block makes its own
 * stream wait for this copy, so a commit to q never runs ahead of its
 * planes.  q in {2, 3, 4}; a q at or below the resident count does nothing.
 *
 * moeq_commit_bits returns MOEQ_ERR_INVALID for a q above the resident
 * count (its planes must be reloaded first).
 *
 * moeq_plane_event — the event recorded after the block's last release or
 * reload copy (owned by the layer; valid until moeq_layer_destroy).
 * moeq_resident_planes, moeq_set_desired_bits, moeq_desired_bits — the
 * page-table state (d in {2, 3, 4}).  Bit-plane layers only
 * (MOEQ_ERR_UNSUPPORTED for INT layers).
 */
moeq_status moeq_plane_release(moeq_layer *L, int32_t expert, int32_t block, void *host,
                               size_t host_bytes, hipStream_t stream);
moeq_status moeq_plane_reload(moeq_layer *L, int32_t expert, int32_t block, int32_t q,
                              const void *host, size_t host_bytes, hipStream_t stream);
moeq_status moeq_plane_event(const moeq_layer *L, int32_t expert, int32_t block, hipEvent_t *ev);
moeq_status moeq_resident_planes(const moeq_layer *L, int32_t expert, int32_t block, int32_t *n);
moeq_status moeq_set_desired_bits(moeq_layer *L, int32_t expert, int32_t block, int32_t d);
moeq_status moeq_desired_bits(const moeq_layer *L, int32_t expert, int32_t block, int32_t *d);
moeq_status moeq_committed_bits(const moeq_layer *L, int32_t expert, int32_t block, int32_t *q);
moeq_status moeq_plane_region(const moeq_layer *L, int32_t expert, int32_t block, int32_t plane,
                              void **ptr, size_t *bytes);

/*
 * moeq_plan_reductions — host-side planner of bit-plane releases ([PW]
 * "What carries the argument": the planner turns a byte target into page
 * releases, taking actions in order of predicted damage per released byte,
 * damage = max(eps, mu_i * g_i * eta_i)).  An action lowers block i's
 * committed bit-plane count by one; while the released bytes are below
 * `target` the available action with the least damage per released byte is
 * taken (ties: lower block index); target <= 0 takes none; q stops at 2.
 *   n blocks; q HOST [n] committed counts in 2..4, overwritten with the plan;
 *   bytes HOST [n][3] page bytes of each block at q = 2, 3, 4 (increasing);
 *   g HOST [n][3] sensitivity of each block at q = 2, 3, 4 (the damage of
 *   an action uses g at the bitwidth it lowers to); mu, eta HOST [n];
 *   eps >= 0; order HOST [max_actions] receives the block of each action
 *   (may be NULL when max_actions is 0); released, damage, n_actions HOST.
 * Pure host code: no device work, no stream.
 */
moeq_status moeq_plan_reductions(int32_t n, int32_t *q, const double *bytes, const double *g,
                                 const double *mu, const double *eta, double eps, double target,
                                 int32_t *order, int32_t max_actions, double *released,
                                 double *damage, int32_t *n_actions);

/* ------------------------------------------------------------- routing -- */

/* Routing outputs, all DEVICE, caller-owned; P = T * k. */
typedef struct {
  int32_t *topk_ids;       /* [T, k] expert ids, by descending logit        */
  float *topk_gates;       /* [T, k] softmax over the k selected logits      */
  int32_t *expert_offsets; /* [E + 1] exclusive prefix sum of expert counts  */
  int32_t *sorted_pairs;   /* [P] pair ids p = t*k + j grouped by expert     */
  int32_t *pair_pos;       /* [P] inverse of sorted_pairs                    */
} moeq_routing;

moeq_status moeq_route_workspace_size(int32_t T, int32_t E, int32_t k, size_t *bytes);

/*
 * moeq_route — top-k routing and the token -> expert counting sort.
 * Per token: the k experts with the largest logits, ordered by descending
 * logit, ties to the lower expert id; gates = softmax over the k selected
 * logits (so they sum to 1).  Then pairs p = t*k + j are counting-sorted by
 * expert: expert_offsets is the exclusive prefix sum of the per-expert pair
 * counts, pairs of one expert are in ascending p, pair_pos inverts
 * sorted_pairs.  ([BEAM] top-k routing with top-n compensation; [MxMoE]
 * uneven expert activation.)
 *   logits DEVICE [T, E] fp32, finite.  T >= 0, 1 <= k <= E <= 256.
 *   ws DEVICE workspace of at least moeq_route_workspace_size bytes (may
 *   be NULL when that size is 0, which it is up to T = 4096; beyond, it
 *   holds per-64-token-segment expert histograms, ceil(T / 64) * E * 4
 *   bytes, so that the sort's work stays linear in T); a smaller one
 *   returns MOEQ_ERR_WORKSPACE.
 */
moeq_status moeq_route(const float *logits, int32_t T, int32_t E, int32_t k,
                       const moeq_routing *out, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * moeq_route_mass — gate-weighted routing mass of every expert from a
 * routing of T tokens: mass[e] = sum of topk_gates over the pairs routed
 * to e ([PW] review summary: the planner's routing-mass buckets protect
 * frequently used experts; the mass is the per-expert usage they bucket),
 * and optionally bucket[e] = number of edges <= mass[e].  fp32, summed in
 * a fixed order (deterministic); the masses of all experts add up to T
 * within rounding.
 *   r      routing of T tokens, top-k, E experts (from moeq_route).
 *   edges  HOST [n_edges] ascending bucket edges, n_edges in 0..8 (NULL if 0).
 *   mass   DEVICE [E] fp32 output.  bucket DEVICE [E] int32 output or NULL.
 */
moeq_status moeq_route_mass(const moeq_routing *r, int32_t T, int32_t E, int32_t k,
                            const float *edges, int32_t n_edges, float *mass, int32_t *bucket,
                            hipStream_t stream);

/* ---------------------------------------------------------- expert FFN -- */

typedef enum {
  MOEQ_PATH_AUTO = 0,   /* chosen from the average tokens per expert          */
  MOEQ_PATH_STREAM = 1, /* weight-streaming: each weight read once per chunk
                           of up to 32 of an expert's tokens (16-row MFMA
                           tiles)                                              */
  /* 2 is reserved (MOEQ_ERR_UNSUPPORTED)                                     */
  MOEQ_PATH_TILED = 3   /* LDS-tiled grouped GEMM for many tokens per expert
                           (INT and bit-plane blocks; MOEQ_ERR_UNSUPPORTED
                           when H is not a multiple of 256, or the rows,
                           codes or compensator width exceed its limits)    */
} moeq_path;

typedef struct {
  int32_t path;    /* moeq_path */
  int32_t split_k; /* down-projection K splits (0 = automatic)               */
} moeq_ffn_options;

/* Workspace bytes moeq_expert_ffn needs for T tokens, top-k and the same
 * options (opts may be NULL). */
moeq_status moeq_ffn_workspace_size(const moeq_layer *L, int32_t T, int32_t k,
                                    const moeq_ffn_options *opts, size_t *bytes);

/*
 * moeq_expert_ffn — the routed expert layer on the packed low-bit weights:
 * for every pair (t, j) with expert e = topk_ids[t][j]
 *   a = L_gate(x_t), b = L_up(x_t), h = SiLU(a) * b, y_pair = L_down(h)
 * with L(v) = W_hat v + comp * (U (V v) + U_G (V_G v)), comp = (j < n_comp)
 * ([BEAM]: compensation for the top-n experts of each token; [MiLo]
 * compensators; [TileQ] shared factors), W_hat = s * (c - z) for INT blocks
 * or LUT[index] for bit-plane blocks ([PW] fused kernel over variable
 * bitwidths), and then y_t = sum_j topk_gates[t][j] * y_pair(t, j) summed in
 * slot order.  Accumulation is fp32; h is rounded to fp16.
 *   x DEVICE [T, H] fp16; r = routing of the same T, k (from moeq_route);
 *   n_comp in 0..k; y DEVICE [T, H] of y_dtype; opts may be NULL.
 */
moeq_status moeq_expert_ffn(const moeq_layer *L, const uint16_t *x, int32_t T,
                            int32_t k, const moeq_routing *r, int32_t n_comp,
                            void *y, int32_t y_dtype, void *ws, size_t ws_bytes,
                            const moeq_ffn_options *opts, hipStream_t stream);

/*
 * moeq_moe_forward — routing and the expert layer in one call: the results
 * of moeq_route into *r followed by moeq_expert_ffn into y, bit for bit
 * (same arguments; logits DEVICE [T, E] fp32).  For decode-sized batches
 * (1 <= T <= 16) of layers with E <= 4 k on the weight-streaming path, the
 * routing, the activation exponents and the gate/up low-rank projection of
 * every (token, expert) pair (which needs no routing) share one launch, one
 * workgroup routing while the others project; other batches run the two calls
 * in order.  ws DEVICE, at least moeq_forward_workspace_size bytes.
 * ([MxMoE] abstract: expert activation; [BEAM] abstract: top-n
 * compensation; the layer of moeq_expert_ffn.)
 */
moeq_status moeq_forward_workspace_size(const moeq_layer *L, int32_t T, int32_t k,
                                        const moeq_ffn_options *opts, size_t *bytes);
moeq_status moeq_moe_forward(const moeq_layer *L, const float *logits, const uint16_t *x,
                             int32_t T, int32_t k, int32_t n_comp, const moeq_routing *r,
                             void *y, int32_t y_dtype, void *ws, size_t ws_bytes,
                             const moeq_ffn_options *opts, hipStream_t stream);

/*
 * moeq_expert_ffn_noalloc — moeq_expert_ffn for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments (minus the workspace), same kernels and bit-identical results;
 * the working memory is a fixed array of moeq_ffn_noalloc_max_bytes bytes
 * (64 MiB) that the library holds in every GPU it runs on until the
 * process ends.  The call allocates nothing (its first call on a device
 * looks up that device's array).  A call whose working memory
 * (moeq_ffn_workspace_size) exceeds the array returns MOEQ_ERR_WORKSPACE
 * before anything is enqueued.  All calls on one GPU share the array:
 * calls that can overlap on one GPU (several streams, several threads)
 * race and must be ordered by the caller.
 */
moeq_status moeq_ffn_noalloc_max_bytes(size_t *bytes);
moeq_status moeq_expert_ffn_noalloc(const moeq_layer *L, const uint16_t *x, int32_t T,
                                    int32_t k, const moeq_routing *r, int32_t n_comp,
                                    void *y, int32_t y_dtype, const moeq_ffn_options *opts,
                                    hipStream_t stream);

/* ---------------------------------------------------------- profiling -- */

/*
 * Per-kernel timing with HIP events recorded around every launch the
 * library makes on the caller's stream.  moeq_profile_enable(1) starts
 * recording (and clears earlier records); moeq_profile_read synchronises the
 * recorded events and returns, for up to max_kernels kernels, their names,
 * launch counts and summed milliseconds.  Host-side state, not thread safe.
 */
moeq_status moeq_profile_enable(int32_t on);
moeq_status moeq_profile_read(int32_t max_kernels, const char **names,
                              int32_t *launches, double *total_ms, int32_t *n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */
