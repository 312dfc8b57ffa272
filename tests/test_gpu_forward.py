"""moeq_moe_forward (routing and the expert layer in one call) gives the
results of moeq_route followed by moeq_expert_ffn bit for bit: on decode
batches that take its fused path (the gate/up projection of every
(token, expert) pair beside the routing, on a second stream), for every
n_comp, on batches and layers that do not, and under HIP graph capture."""

import numpy as np
import pytest

from synth import configs, gen
from tests import layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = {
    "tiny_t16": ("tiny", dict(T=16)),                      # E 8, k 2: fused
    "decode": ("decode", dict(H=512, I=1792)),            # fused (int3, G128, outliers)
    "decode_t1": ("decode", dict(H=512, I=1792, T=1)),    # fused, one token
    "tiny_t64": ("tiny", {}),                             # more than 16 tokens: route, then FFN
    "finegrained": ("finegrained", dict(T=16)),           # E 64 > 4 k: route, then FFN
    # fused, with shared factors (groups of 2) large in the output
    "tiny_shared": ("tiny", dict(T=16, rs=16, share=2, factor_std=0.05)),
    # a long batch: the routing's workspace follows the FFN's in ws
    "tiny_t4160": ("tiny", dict(T=4160)),
}
_cache = {}


def _setup(case):
    if case not in _cache:
        name, over = CASES[case]
        cfg = configs.reduced(configs.get(name), **over)
        orc = layers.oracle_layer(cfg, 0, cache_blocks=3 * cfg["E"])
        _cache.clear()
        _cache[case] = (cfg, orc, layers.device_layer(cfg, 0, orc))
    return _cache[case]


@pytest.mark.parametrize("case", list(CASES))
def test_forward_equals_route_then_ffn(case):
    from bit_quantized_moe_token_amd import moeq
    cfg, orc, dev = _setup(case)
    x = torch.from_numpy(gen.gen_x(cfg, 0)).cuda()
    logits = torch.from_numpy(gen.gen_logits(cfg, 0)).cuda()
    k = cfg["k"]
    for n_comp in sorted({0, 1, cfg["n_comp"], k}):
        rt = moeq.route(logits, k)
        ref = moeq.expert_ffn(dev, x, rt, n_comp, out_dtype=torch.float32)
        y, rf = moeq.moe_forward(dev, logits, x, k, n_comp, out_dtype=torch.float32)
        torch.cuda.synchronize()
        for name in ("ids", "gates", "offsets", "sorted_pairs", "pair_pos"):
            assert torch.equal(getattr(rf, name), getattr(rt, name)), f"{case} n_comp={n_comp}: routing {name}"
        assert torch.equal(y, ref), f"{case} n_comp={n_comp}: output differs from route + expert_ffn"
    layers.check_y(y.cpu().numpy(), layers.oracle_y(orc, cfg, gen.gen_x(cfg, 0), gen.gen_logits(cfg, 0), k),
                   case + " forward")


def test_forward_graph_replay():
    """The fused call's fork and join are captured into a HIP graph; every
    replay gives the eager result, with eager work between replays."""
    from bit_quantized_moe_token_amd import moeq
    cfg, orc, dev = _setup("decode")
    x = torch.from_numpy(gen.gen_x(cfg, 0)).cuda()
    logits = torch.from_numpy(gen.gen_logits(cfg, 0)).cuda()
    k, T = cfg["k"], cfg["T"]
    rt = moeq.RoutingOut(T, cfg["E"], k, x.device)
    ws = moeq.FfnWorkspace(dev, T, k, forward=True)
    y = torch.empty((T, cfg["H"]), dtype=torch.float16, device=x.device)

    def step():
        moeq.moe_forward(dev, logits, x, k, cfg["n_comp"], routing=rt, out=y, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for it in range(4):
        y.zero_()
        rt.sorted_pairs.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {it} differs from the eager call"
        other, _ = moeq.moe_forward(dev, torch.flip(logits, [0]).contiguous(), torch.flip(x, [0]).contiguous(), k,
                                    cfg["n_comp"])
        torch.cuda.synchronize()
