"""Workload shapes for the routed low-bit MoE expert layer.

Five seeded synthetic layers stand in for the trained MoE models the pages
evaluate on (Mixtral-8x7B-shaped layers and fine-grained many-expert layers;
PagedWeight review, "Summary" of the referee report, names Qwen1.5-MoE-A2.7B,
Mixtral-8x7B and Gemma-4-26B-A4B).  No trained weights or datasets are used.

Each config is a plain dict.  Keys:
  name, T (tokens), E (experts), k (top-k), H (hidden), I (intermediate),
  fmt ("int" | "bitplane"), G (quantization group along K),
  bits (int, or None when drawn per block from bits_choices/bits_probs),
  r (per-expert compensator rank), rs (shared rank), share (experts per
  shared-factor group), comp ("svd" | "random"), n_comp (leading top-k slots
  that get compensation), outlier_frac / outlier_mult (activation outliers),
  zipf (exponent of the per-expert router bias, or None).

This module holds shapes only; it contains none of the method's arithmetic.
"""

import copy

TINY = dict(
    name="tiny_e8_h256_i512_t64_int4_g64_svd16",
    T=64, E=8, k=2, H=256, I=512,
    fmt="int", G=64, bits=4, bits_choices=None, bits_probs=None,
    r=16, rs=0, share=0, comp="svd", n_comp=2,
    outlier_frac=0.0, outlier_mult=1.0, zipf=None,
)

MIXTRAL_DECODE = dict(
    name="mixtral_e8_h4096_i14336_t16_int3_g128_r32_decode",
    T=16, E=8, k=2, H=4096, I=14336,
    fmt="int", G=128, bits=3, bits_choices=None, bits_probs=None,
    r=32, rs=0, share=0, comp="random", n_comp=2,
    outlier_frac=0.01, outlier_mult=20.0, zipf=1.1,
)

MIXTRAL_PREFILL = dict(
    name="mixtral_e8_h4096_i14336_t4096_int4_g128_r32_prefill",
    T=4096, E=8, k=2, H=4096, I=14336,
    fmt="int", G=128, bits=4, bits_choices=None, bits_probs=None,
    r=32, rs=0, share=0, comp="random", n_comp=2,
    outlier_frac=0.01, outlier_mult=20.0, zipf=1.1,
)

FINE_GRAINED = dict(
    name="finegrained_e64_k6_h2048_i1408_t256_mixed234_g64_r16_top2comp",
    T=256, E=64, k=6, H=2048, I=1408,
    fmt="int", G=64, bits=None, bits_choices=(2, 3, 4), bits_probs=(0.3, 0.4, 0.3),
    r=16, rs=0, share=0, comp="random", n_comp=2,
    outlier_frac=0.0, outlier_mult=1.0, zipf=None,
)

BITPLANE = dict(
    name="bitplane_e128_k8_h2048_i768_t512_q234_g128_shared32_r8",
    T=512, E=128, k=8, H=2048, I=768,
    fmt="bitplane", G=128, bits=None, bits_choices=(2, 3, 4), bits_probs=(0.3, 0.4, 0.3),
    r=8, rs=32, share=4, comp="random", n_comp=8,
    outlier_frac=0.0, outlier_mult=1.0, zipf=None,
)

CONFIGS = [TINY, MIXTRAL_DECODE, MIXTRAL_PREFILL, FINE_GRAINED, BITPLANE]
BY_NAME = {c["name"]: c for c in CONFIGS}
SHORT = {"tiny": TINY, "decode": MIXTRAL_DECODE, "prefill": MIXTRAL_PREFILL,
         "finegrained": FINE_GRAINED, "bitplane": BITPLANE}


def get(name):
    """Return a deep copy of a config by short or full name."""
    if name in SHORT:
        return copy.deepcopy(SHORT[name])
    return copy.deepcopy(BY_NAME[name])


def reduced(cfg, **over):
    """Same structure with smaller dimensions (for fast parity runs)."""
    c = copy.deepcopy(cfg)
    c.update(over)
    c["name"] = cfg["name"] + "_reduced_" + "_".join(f"{k}{v}" for k, v in sorted(over.items()))
    return c
