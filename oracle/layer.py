"""A quantized MoE layer for the oracle, built lazily from fp16 weights with
the oracle's own PTQ (test infrastructure only; see ``oracle/__init__.py``).

The layer exposes what ``forward.expert_ffn`` reads:
  qblock(e, blk, rows=None)  quantized block (INT codes/s16/z, or bit-plane
                             parent codes c4 + LUT + committed q)
  factors(e, blk)            per-expert (U, V) fp16 or None
  shared(g, blk)             shared (U_G, V_G) fp16 of expert group g or None
  group_of(e)                expert group index (contiguous groups of `share`)
"""

from collections import OrderedDict

import numpy as np

from . import forward, ptq


class OracleLayer:
    def __init__(self, E, H, I, G, fmt, bits, weight_rows, factors=None,
                 shared=None, share=0, svd_rank=0, cache_blocks=8):
        """weight_rows(e, blk, rows) -> fp16 [len(rows) or N, K] (rows=None: all).
        bits: [E, 3] INT bitwidth b or committed bit-plane q per block.
        factors(e, blk) / shared(g, blk) -> (U16, V16) or None.
        svd_rank > 0 replaces per-expert factors by the truncated SVD of each
        block's quantization residual."""
        self.E, self.H, self.I, self.G = E, H, I, G
        self.fmt = fmt
        self.bits = np.asarray(bits, dtype=np.uint8)
        self._weight_rows = weight_rows
        self._factors = factors
        self._shared = shared
        self.share = share
        self.svd_rank = svd_rank
        self._cache = OrderedDict()
        self._cache_blocks = cache_blocks
        self._svd = {}

    def group_of(self, e):
        return e // self.share if self.share else 0

    def _quantize(self, W16, e, blk):
        b = int(self.bits[e, blk])
        if self.fmt == "int":
            codes, s16, z = ptq.rtn_quantize(W16, b, self.G)
            return dict(fmt="int", codes=codes, s16=s16, z=z, b=b)
        c4, s16, z = ptq.rtn_quantize(W16, 4, self.G)
        lut = ptq.bitplane_lut(W16, c4, s16, z, b, self.G)
        return dict(fmt="bitplane", c4=c4, lut=lut, q=b, s16=s16, z=z)

    def qblock(self, e, blk, rows=None):
        if rows is not None:
            W16 = self._weight_rows(e, blk, np.asarray(rows))
            return self._quantize(W16, e, blk)
        key = (e, blk)
        if key in self._cache:
            self._cache.move_to_end(key)
            return self._cache[key]
        qb = self._quantize(self._weight_rows(e, blk, None), e, blk)
        if self._cache_blocks:
            self._cache[key] = qb
            while len(self._cache) > self._cache_blocks:
                self._cache.popitem(last=False)
        return qb

    def factors(self, e, blk):
        if self.svd_rank > 0:
            key = (e, blk)
            if key not in self._svd:
                W16 = self._weight_rows(e, blk, None)
                W_hat = forward.dequant_block(self.qblock(e, blk), self.G)
                U16, V16, _, _, _ = ptq.svd_compensator(W16, W_hat, self.svd_rank)
                self._svd[key] = (U16, V16)
            return self._svd[key]
        return self._factors(e, blk) if self._factors else None

    def shared(self, g, blk):
        return self._shared(g, blk) if self._shared else None
