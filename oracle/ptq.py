"""Oracle PTQ: the encoding of expert weights (test infrastructure only).

Readings of the pages (none of them prints the quantizer; see the header of
``oracle/__init__.py`` for who may use this module):

* Asymmetric round-to-nearest group quantization (MiLo abstract: extreme,
  under-4-bit quantization of MoE experts; MxMoE abstract: bitwidth chosen per
  linear block).  Per row n and per group g of G consecutive columns:
      lo = min(0, min w),  hi = max(0, max w)
      s16 = fp16((hi - lo) / (2^b - 1))   (one rounding, half-to-even;
                                            s16 = 1 when hi == lo or s16 == 0)
      z   = clamp(rint(-lo / s16), 0, 2^b - 1)
      c   = clamp(rint(w / s16) + z, 0, 2^b - 1)
  with rint = round half to even, all in float64 on the fp16 values.
* Bit-plane + lookup-table form (PagedWeight, Figure 3 caption: a shared
  bit-plane format where subsets of planes give the bitwidths, with a LUT of
  bitwidth-specific centroid values).  Parent codes are the 4-bit RTN codes
  c4 (planes P3 = MSB .. P0); a block committed to q bits uses the top q
  planes, index i = c4 >> (4 - q).  LUT slot j < 2^q holds the centroid of the
  group's weights with index j: fp16(mean), or, for an empty bucket, the value
  at the middle of the bucket's code range, fp16(s16 * (j * 2^(4-q) +
  (2^(4-q) - 1) / 2 - z)).  Slots j >= 2^q are zero.
* Low-rank compensator (MiLo abstract: low-rank compensators recover the loss
  of extreme quantization): truncated SVD of the residual R = W - W_hat,
  R ~ P_r S_r Q_r^T, U = P_r S_r^(1/2), V = S_r^(1/2) Q_r^T, stored fp16.
"""

import numpy as np


def to_f16(a):
    """Round float64 values to fp16 once, half to even (numpy converts double
    to half directly, without passing through float32)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def rtn_quantize(W16, b, G):
    """Asymmetric RTN of an fp16 block [N, K] with b bits and groups of G along K.

    Returns (codes uint8 [N, K], s16 float16 [N, K/G], z uint8 [N, K/G]).
    """
    W16 = np.asarray(W16)
    assert W16.dtype == np.float16 and W16.ndim == 2
    N, K = W16.shape
    assert K % G == 0 and b in (2, 3, 4)
    qmax = float(2 ** b - 1)
    Wg = W16.astype(np.float64).reshape(N, K // G, G)
    lo = np.minimum(0.0, Wg.min(axis=-1))
    hi = np.maximum(0.0, Wg.max(axis=-1))
    s16 = to_f16((hi - lo) / qmax)
    s16[(hi == lo) | (s16 == 0)] = np.float16(1.0)
    s = s16.astype(np.float64)
    z = np.clip(np.rint(-lo / s), 0.0, qmax)
    c = np.clip(np.rint(Wg / s[..., None]) + z[..., None], 0.0, qmax)
    return c.reshape(N, K).astype(np.uint8), s16, z.astype(np.uint8)


def bitplane_index(c4, q):
    """Index formed by the top q of the four bit-planes of 4-bit codes."""
    return (np.asarray(c4, dtype=np.uint8) >> (4 - q)).astype(np.uint8)


def bitplane_lut(W16, c4, s16, z, q, G):
    """Per-(row, group) 16-slot fp16 LUT for a block committed to q bits.

    Slot j < 2^q: fp16 of the mean of the group's weights whose index is j
    (empty bucket: fp16 of the bucket's mid-code value); slots >= 2^q are 0.
    Returns float16 [N, K/G, 16].
    """
    W16 = np.asarray(W16)
    N, K = W16.shape
    ng = K // G
    nq = 2 ** q
    span = 2 ** (4 - q)
    mid = np.arange(nq, dtype=np.float64) * span + (span - 1) / 2.0
    lut = np.zeros((N, ng, 16), dtype=np.float16)
    for r0 in range(0, N, 512):                       # row chunks bound memory
        r1 = min(N, r0 + 512)
        idx = bitplane_index(c4[r0:r1], q).reshape(r1 - r0, ng, G)
        W = W16[r0:r1].astype(np.float64).reshape(r1 - r0, ng, G)
        onehot = (idx[..., None] == np.arange(nq, dtype=np.uint8)).astype(np.float64)
        sums = np.einsum("ngk,ngkj->ngj", W, onehot)  # exact: sums of fp16 values
        counts = onehot.sum(axis=2)
        fallback = (s16[r0:r1].astype(np.float64)[..., None]
                    * (mid[None, None, :] - z[r0:r1].astype(np.float64)[..., None]))
        with np.errstate(invalid="ignore", divide="ignore"):
            mean = sums / counts
        lut[r0:r1, :, :nq] = to_f16(np.where(counts > 0, mean, fallback))
    return lut


def mean_residual_compensator(W16_list, W_hat_list, r):
    """Rank-r factor pair shared by n blocks (TileQ abstract: factors shared
    across experts): the truncated SVD of the mean residual
    R = (1/n) sum_m (W_m - W_hat_m).  It minimizes sum_m ||R_m - U V||_F^2
    over rank-r U V, since sum_m ||R_m - X||^2 = sum_m ||R_m - R||^2 +
    n ||R - X||^2.  Same return values and split as svd_compensator; n = 1
    is svd_compensator itself.
    """
    Rm = [np.asarray(W, dtype=np.float64) - np.asarray(Wh, dtype=np.float64) for W, Wh in zip(W16_list, W_hat_list)]
    mean = sum(Rm) / len(Rm)
    return svd_compensator(mean, np.zeros_like(mean), r)


def svd_compensator(W16, W_hat, r):
    """Rank-r compensator of the quantization residual R = W - W_hat.

    Returns (U16 [N, r], V16 [r, K], U64, V64, sigma) where U64 @ V64 is the
    best rank-r approximation of R in float64, split evenly (S^(1/2) on both
    sides), and sigma are all singular values of R.
    """
    R = np.asarray(W16, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    P, S, Qt = np.linalg.svd(R, full_matrices=False)
    root = np.sqrt(S[:r])
    U64 = P[:, :r] * root[None, :]
    V64 = root[:, None] * Qt[:r, :]
    return U64.astype(np.float16), V64.astype(np.float16), U64, V64, S
