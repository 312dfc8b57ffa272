"""GPU parity across the fp16 range: the same seeded layers with the
activations scaled by 2^-12 .. 2^4 (and one layer whose weights, and so its
h, are 16 times smaller), on every kernel path: weight streaming with INT
codes of 2, 3 and 4 bits in groups of 64 and 128, the tiled path, mixed
per-block bitwidths and the bit-plane form.  The tolerance is the one of
every other parity test; y is compared in fp32 (an fp16 output cannot hold
the smallest of these results)."""

import numpy as np
import pytest

from synth import configs, gen
from tests import layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCALES = [2.0 ** -12, 2.0 ** -10, 2.0 ** -8, 1.0, 2.0 ** 4]
PATH_AUTO, PATH_STREAM, PATH_TILED = 0, 1, 3

# name -> (base config, overrides, forced path)
CASES = {
    "stream_b2_g64": ("decode", dict(H=512, I=1792, bits=2, G=64), PATH_STREAM),
    "stream_b2_g128": ("decode", dict(H=512, I=1792, bits=2, G=128), PATH_STREAM),
    "stream_b3_g64": ("decode", dict(H=512, I=1792, bits=3, G=64), PATH_STREAM),
    "stream_b3_g128": ("decode", dict(H=512, I=1792, bits=3, G=128), PATH_STREAM),
    "stream_b4_g64": ("decode", dict(H=512, I=1792, bits=4, G=64), PATH_STREAM),
    "stream_b4_g128": ("decode", dict(H=512, I=1792, bits=4, G=128), PATH_STREAM),
    # 32-token chunks (two MFMA token tiles per chunk)
    "stream_b3_g128_t80": ("decode", dict(H=512, I=1792, T=80), PATH_STREAM),
    "tiled_b4": ("prefill", dict(H=512, I=1792, T=512), PATH_TILED),
    "tiled_b3": ("decode", dict(H=512, I=1792, T=512), PATH_TILED),
    # gate and up of different bitwidths in one workgroup, group 64
    "mixed_bits": ("finegrained", dict(E=16, T=64), PATH_AUTO),
    "bitplane": ("bitplane", dict(E=32, T=128), PATH_AUTO),
}

_layers = {}


def _layer(case, w_scale=1.0):
    key = (case, w_scale)
    if key not in _layers:
        name, over, path = CASES[case]
        over = dict(over)
        if w_scale != 1.0:
            over["w_scale"] = w_scale
        cfg = configs.reduced(configs.get(name), **over)
        orc = layers.oracle_layer(cfg, 0, cache_blocks=3 * cfg["E"])
        dev = layers.device_layer(cfg, 0, orc)
        _layers[key] = (cfg, orc, dev, path)
    return _layers[key]


def _check(case, x_scale, w_scale=1.0):
    from bit_quantized_moe_token_amd import moeq
    cfg, orc, dev, path = _layer(case, w_scale)
    c = dict(cfg, x_scale=x_scale)
    x = gen.gen_x(c, 0)
    logits = gen.gen_logits(c, 0)
    rt = moeq.route(torch.from_numpy(logits).cuda(), c["k"])
    y = moeq.expert_ffn(dev, torch.from_numpy(x).cuda(), rt, c["n_comp"], out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    ref = layers.oracle_y(orc, c, x, logits, c["n_comp"])
    rel, fro = layers.check_y(y.cpu().numpy(), ref, f"{case} x_scale={x_scale:g} w_scale={w_scale:g}")
    print(f"{case} x*{x_scale:g} w*{w_scale:g}: max|err|/rms {rel:.2e} fro {fro:.2e}")


@pytest.mark.parametrize("scale", SCALES, ids=lambda s: f"x{np.log2(s):+.0f}")
@pytest.mark.parametrize("case", list(CASES))
def test_parity_across_activation_scale(case, scale):
    _check(case, scale)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -8], ids=lambda s: f"x{np.log2(s):+.0f}")
@pytest.mark.parametrize("case", ["stream_b3_g128", "stream_b4_g64", "tiled_b4", "bitplane"])
def test_parity_small_h(case, scale):
    """Weights 16 times smaller: h about 256 times smaller than usual."""
    _check(case, scale, w_scale=2.0 ** -4)
