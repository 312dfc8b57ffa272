"""Seeded synthetic inputs for the routed low-bit MoE expert layer.

Every random quantity is drawn from numpy ``default_rng`` with its own stream
key, so that changing T (or drawing fewer rows) never shifts any other draw:

  [seed, 0]                      router logits  N(0, 1)
  [seed, 1]                      activations x  N(0, 1)
  [seed, 2, e, blk, chunk]       expert weights N(0, 0.02), 256-row chunks
  [seed, 3]                      per-block bitwidths (mixed-precision configs)
  [seed, 4, e, blk, 0|1]         per-expert compensator factors U | V, N(0, 0.01)
  [seed, 5]                      Zipf permutation of experts (router bias)
  [seed, 6]                      outlier activation channels
  [seed, 7, grp, blk, 0|1]       shared compensator factors U | V, N(0, 0.01)
  [seed, 8, e, blk]              Gaussian test matrix of the compensator fit, N(0, 1)

"N(0, s)" is read as mean 0 and standard deviation s.  Optional config keys
change a layer without changing any draw: x_scale multiplies the activations
and w_scale the expert weights (both move a layer across the fp16 range),
and factor_std replaces the 0.01 of the random compensator factors (larger
values make the low-rank terms a large part of the output); each is applied
before the rounding to fp16.  Blocks are numbered
0 = gate, 1 = up, 2 = down; gate/up blocks are [I, H] (rows = outputs), down
is [H, I].  Values are rounded to the storage type (fp16 weights, activations
and factors, fp32 logits) here, and those rounded values are the inputs of
both the oracle and the device path.

This module draws random numbers only; it holds none of the method's
arithmetic (no quantization, routing or expert computation).
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROW_CHUNK = 256
GATE, UP, DOWN = 0, 1, 2


def _rng(*key):
    return np.random.default_rng(list(key))


def block_shape(cfg, blk):
    """(N, K) of a block: gate/up map H -> I, down maps I -> H."""
    if blk in (GATE, UP):
        return cfg["I"], cfg["H"]
    return cfg["H"], cfg["I"]


def _weight_chunk(cfg, seed, e, blk, chunk):
    n, kdim = block_shape(cfg, blk)
    r0 = chunk * ROW_CHUNK
    rows = min(ROW_CHUNK, n - r0)
    a = _rng(seed, 2, e, blk, chunk).standard_normal((rows, kdim), dtype=np.float32)
    a *= np.float32(0.02 * float(cfg.get("w_scale", 1.0)))
    return a.astype(np.float16)


def _pool_size():
    return max(1, min(16, os.cpu_count() or 1))


def gen_weight_block(cfg, seed, e, blk, threads=None):
    """Full fp16 weight block [N, K] of expert e, block blk."""
    n, kdim = block_shape(cfg, blk)
    nchunks = (n + ROW_CHUNK - 1) // ROW_CHUNK
    out = np.empty((n, kdim), dtype=np.float16)

    def fill(c):
        out[c * ROW_CHUNK:c * ROW_CHUNK + ROW_CHUNK] = _weight_chunk(cfg, seed, e, blk, c)

    threads = threads or _pool_size()
    if nchunks == 1 or threads == 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def gen_weight_rows(cfg, seed, e, blk, rows):
    """Selected rows of a weight block, identical to gen_weight_block(...)[rows]."""
    rows = np.asarray(rows, dtype=np.int64)
    _, kdim = block_shape(cfg, blk)
    out = np.empty((len(rows), kdim), dtype=np.float16)
    cache = {}
    for i, r in enumerate(rows):
        c = int(r) // ROW_CHUNK
        if c not in cache:
            cache[c] = _weight_chunk(cfg, seed, e, blk, c)
        out[i] = cache[c][int(r) - c * ROW_CHUNK]
    return out


def zipf_bias(cfg, seed):
    """Per-expert router bias: log of Zipf(s) probabilities over a seeded expert
    ranking (bias_e = -s * ln(rank_e), rank_e in 1..E); zeros when unused."""
    E = cfg["E"]
    if not cfg.get("zipf"):
        return np.zeros(E, dtype=np.float64)
    rank = 1 + _rng(seed, 5).permutation(E)
    return -float(cfg["zipf"]) * np.log(rank.astype(np.float64))


def gen_logits(cfg, seed):
    """Router logits [T, E] fp32: N(0,1) plus the per-expert bias, summed in fp64."""
    T, E = cfg["T"], cfg["E"]
    l = _rng(seed, 0).standard_normal((T, E))
    l = l + zipf_bias(cfg, seed)[None, :]
    return l.astype(np.float32)


def outlier_channels(cfg, seed):
    """Sorted indices of the outlier channels: round(frac * H) of them."""
    H = cfg["H"]
    n = int(round(cfg.get("outlier_frac", 0.0) * H))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed, 6).choice(H, size=n, replace=False))


def gen_x(cfg, seed):
    """Activations [T, H] fp16: N(0,1), outlier channels scaled before rounding."""
    T, H = cfg["T"], cfg["H"]
    x = _rng(seed, 1).standard_normal((T, H))
    ch = outlier_channels(cfg, seed)
    if len(ch):
        x[:, ch] *= float(cfg["outlier_mult"])
    x *= float(cfg.get("x_scale", 1.0))
    return x.astype(np.float16)


def gen_bits(cfg, seed):
    """Per-(expert, block) bitwidth [E, 3] uint8 (INT b, or committed bit-plane q)."""
    E = cfg["E"]
    if cfg.get("bits") is not None:
        return np.full((E, 3), int(cfg["bits"]), dtype=np.uint8)
    ch = np.asarray(cfg["bits_choices"], dtype=np.uint8)
    p = np.asarray(cfg["bits_probs"], dtype=np.float64)
    return _rng(seed, 3).choice(ch, size=(E, 3), p=p).astype(np.uint8)


def gen_factors(cfg, seed, e, blk):
    """Random per-expert compensator (U [N, r], V [r, K]) fp16, or None if r == 0."""
    r = cfg.get("r", 0)
    if r == 0:
        return None
    n, kdim = block_shape(cfg, blk)
    sd = cfg.get("factor_std", 0.01)
    U = (_rng(seed, 4, e, blk, 0).standard_normal((n, r)) * sd).astype(np.float16)
    V = (_rng(seed, 4, e, blk, 1).standard_normal((r, kdim)) * sd).astype(np.float16)
    return U, V


def gen_shared_factors(cfg, seed, grp, blk):
    """Random shared compensator of expert group grp, or None if rs == 0."""
    rs = cfg.get("rs", 0)
    if rs == 0:
        return None
    n, kdim = block_shape(cfg, blk)
    sd = cfg.get("factor_std", 0.01)
    U = (_rng(seed, 7, grp, blk, 0).standard_normal((n, rs)) * sd).astype(np.float16)
    V = (_rng(seed, 7, grp, blk, 1).standard_normal((rs, kdim)) * sd).astype(np.float16)
    return U, V


def gen_test_matrix(cfg, seed, e, blk, l):
    """Gaussian test matrix [K, l] fp32 of the randomized compensator fit of
    block (e, blk) (K = the block's input dimension)."""
    _, kdim = block_shape(cfg, blk)
    return _rng(seed, 8, e, blk).standard_normal((kdim, l)).astype(np.float32)


def n_groups(cfg):
    share = cfg.get("share", 0)
    if not share:
        return 0
    return math.ceil(cfg["E"] / share)
