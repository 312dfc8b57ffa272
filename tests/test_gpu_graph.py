"""A captured HIP graph of one routed-layer step (routing + expert FFN, as
the benchmark replays it) gives the eager result bit for bit on every
replay, with eager work and synchronisations between the replays."""

import numpy as np
import pytest

from synth import configs, gen
from tests import layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over", [("decode", dict(H=512, I=1792)),
                                       ("prefill", dict(H=512, I=1792, T=1024))])
def test_graph_replay_equals_eager(name, over):
    from bit_quantized_moe_token_amd import moeq
    cfg = configs.reduced(configs.get(name), **over)
    dev = layers.device_layer(cfg, 0)
    x = torch.from_numpy(gen.gen_x(cfg, 0)).cuda()
    logits = torch.from_numpy(gen.gen_logits(cfg, 0)).cuda()
    k, T = cfg["k"], cfg["T"]
    rt = moeq.RoutingOut(T, cfg["E"], k, x.device)
    ws = moeq.FfnWorkspace(dev, T, k)
    y = torch.empty((T, cfg["H"]), dtype=torch.float16, device=x.device)

    def step():
        moeq.route(logits, k, out=rt)
        moeq.expert_ffn(dev, x, rt, cfg["n_comp"], out=y, ws=ws)

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
        assert torch.equal(y, eager), f"replay {it} differs from the eager step"
        # eager work between replays, on other inputs
        other = moeq.route(torch.flip(logits, [0]).contiguous(), k)
        moeq.expert_ffn(dev, torch.flip(x, [0]).contiguous(), other, cfg["n_comp"])
        torch.cuda.synchronize()
