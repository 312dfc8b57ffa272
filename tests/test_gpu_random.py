"""GPU parity of the routed expert layer on seeded random shapes: expert
count, top-k, hidden and intermediate sizes (any multiple of 128, including
a single 128-column tile and ragged groups of K tiles), token count, INT
(groups of 64 or 128) or bit-plane blocks with per-block bitwidths,
per-expert and shared compensator ranks, the number of compensated slots
and the kernel path (default, streaming, tiled where the shape allows it),
each against the fp64 oracle at the same tolerance as the fixed workloads;
and, where the fused call applies, moeq_moe_forward equal to routing then
the expert layer bit for bit."""

import numpy as np
import pytest

from synth import configs, gen
from tests import layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PATH_AUTO, PATH_STREAM, PATH_TILED = 0, 1, 3


def _tiled_fits(c):
    rz = -(-c["r"] // 32) * 32 + -(-c["rs"] // 32) * 32
    return c["H"] % 256 == 0 and 2 * rz <= 136


def _cases(n=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        fmt = "bitplane" if rng.random() < 0.4 else "int"
        E = int(rng.choice([2, 3, 5, 8, 16, 24]))
        H = int(rng.choice([128, 256, 384, 512, 768, 1024]))
        I = int(rng.choice([128, 256, 384, 640, 896]))
        if E * H * I > 8 * 2 ** 20:
            continue
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 2, 9, 17, 40, 100, 260, 600]))
        G = 128 if fmt == "bitplane" else int(rng.choice([64, 128]))
        fixed = rng.random() < 0.3
        r = int(rng.choice([0, 8, 16, 24, 32]))
        rs = int(rng.choice([0, 0, 8, 16, 32]))
        share = min(int(rng.choice([2, 3, 4])), E) if rs else 0   # experts per group, 1..E
        c = dict(configs.get("finegrained"), T=T, E=E, k=k, H=H, I=I, fmt=fmt, G=G,
                 bits=int(rng.choice([2, 3, 4])) if fixed else None,
                 bits_choices=(2, 3, 4), bits_probs=(1 / 3, 1 / 3, 1 / 3),
                 r=r, rs=rs, share=share, comp="random", n_comp=int(rng.integers(0, k + 1)),
                 outlier_frac=float(rng.choice([0.0, 0.01])), outlier_mult=20.0,
                 zipf=None if rng.random() < 0.5 else 1.1)
        c["name"] = (f"random{len(out)}_{fmt}_e{E}_k{k}_h{H}_i{I}_t{T}_g{G}_r{r}_rs{rs}x{share}"
                     f"_nc{c['n_comp']}")
        paths = [PATH_AUTO, PATH_STREAM] + ([PATH_TILED] * 3 if _tiled_fits(c) else [])
        c["path"] = int(rng.choice(paths))
        out.append(c)
    return out


CASES = _cases()


@pytest.mark.parametrize("cfg", CASES, ids=[c["name"] for c in CASES])
def test_random_shape_matches_oracle(cfg):
    from bit_quantized_moe_token_amd import moeq
    print(f"case {cfg['name']} path {cfg['path']}", flush=True)
    orc = layers.oracle_layer(cfg, 0, cache_blocks=3 * cfg["E"])
    dev = layers.device_layer(cfg, 0, orc)
    x, logits = gen.gen_x(cfg, 0), gen.gen_logits(cfg, 0)
    xd, ld = torch.from_numpy(x).cuda(), torch.from_numpy(logits).cuda()
    rt = moeq.route(ld, cfg["k"])
    y = moeq.expert_ffn(dev, xd, rt, cfg["n_comp"], out_dtype=torch.float32, path=cfg["path"])
    torch.cuda.synchronize()
    ref = layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"])
    rel, fro = layers.check_y(y.cpu().numpy(), ref, cfg["name"])
    print(f"  max|err|/rms {rel:.2e}  fro {fro:.2e}")
    # routing then the layer, and the one-call forward, agree bit for bit
    yf, _ = moeq.moe_forward(dev, ld, xd, cfg["k"], cfg["n_comp"], out_dtype=torch.float32, path=cfg["path"])
    torch.cuda.synchronize()
    assert torch.equal(yf, y)
