"""GPU parity at full size in the launch configuration the benchmark times:
the Mixtral-shaped layers (H 4096, I 14336, 8 experts, top-2) and the
bit-plane layer with shared factors (128 experts, top-8, 512 tokens, all
4096 pairs routed).  The whole layer is quantized and packed by the
library, routed and evaluated for the whole batch, and the oracle
recomputes sampled outputs one by one (every gate/up row of the sampled
tokens' experts, the down rows of the sampled output columns) from its own
quantization of the same fp16 weights."""

import numpy as np
import pytest

from synth import configs, gen
from tests import layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _sample_cols(H, n, seed):
    rng = np.random.default_rng([seed, 99])
    cols = set(rng.choice(H, size=n, replace=False).tolist())
    cols |= {0, 1, 127, 128, H - 129, H - 1}          # first/last tiles and strip edges
    return np.array(sorted(cols))


def _run_full(name, tokens, n_cols, seed=0, path=0, T=None):
    from bit_quantized_moe_token_amd import moeq
    cfg = configs.get(name)
    if T is not None:
        cfg = dict(cfg, T=T)
    x = gen.gen_x(cfg, seed)
    logits = gen.gen_logits(cfg, seed)
    dev = layers.device_layer(cfg, seed)
    xd = torch.from_numpy(x).cuda()
    rt = moeq.route(torch.from_numpy(logits).cuda(), cfg["k"])
    y = moeq.expert_ffn(dev, xd, rt, cfg["n_comp"], out_dtype=torch.float16, path=path)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    del dev
    torch.cuda.empty_cache()
    cols = _sample_cols(cfg["H"], n_cols, seed)
    orc = layers.oracle_layer(cfg, seed, cache_blocks=2 * cfg["E"])
    ref = layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"], tokens=tokens, cols=cols)
    rel, fro = layers.check_y(y[np.ix_(tokens, cols)], ref, name)
    print(f"{name} full size (path {path}), {len(tokens)} tokens x {len(cols)} columns: "
          f"max|err|/rms {rel:.2e}  fro {fro:.2e}")


@pytest.mark.timeout(600)
def test_decode_full_size_sampled():
    """Mixtral decode: 16 tokens, int3 G128, rank 32 (all tokens checked)."""
    _run_full("decode", np.arange(16), 384)


@pytest.mark.timeout(600)
def test_prefill_full_size_sampled():
    """Mixtral prefill: 4096 tokens, int4 G128, rank 32; tokens sampled
    across the batch, including the first and the last."""
    T = configs.get("prefill")["T"]
    tokens = np.unique(np.concatenate([[0, 1, T - 1], np.linspace(0, T - 1, 7).astype(int)]))
    _run_full("prefill", tokens, 256)


@pytest.mark.timeout(600)
def test_bitplane_full_size_sampled():
    """Bit-plane layer: 128 experts, top-8, 512 tokens (4096 pairs), q per
    block in {2, 3, 4}, shared rank-32 factors per 4 experts plus rank-8
    per expert; tokens sampled across the batch."""
    T = configs.get("bitplane")["T"]
    tokens = np.unique(np.concatenate([[0, 1, T - 1], np.linspace(0, T - 1, 6).astype(int)]))
    _run_full("bitplane", tokens, 256)


@pytest.mark.timeout(600)
def test_bitplane_full_size_sampled_tiled():
    """The same bit-plane layer on the tiled path (forced): 128-token tiles
    of the bit-plane blocks at every committed q, shared factors."""
    T = configs.get("bitplane")["T"]
    tokens = np.unique(np.concatenate([[0, 2, T - 2], np.linspace(0, T - 1, 5).astype(int)]))
    _run_full("bitplane", tokens, 192, path=3)


@pytest.mark.timeout(600)
def test_bitplane_prefill_full_size_sampled():
    """The bit-plane layer with 4096 tokens (256 pairs per expert on
    average), as the benchmark runs it: the default path is the tiled one
    (three 128-token tiles for most experts, the last one partial)."""
    T = 4096
    tokens = np.unique(np.concatenate([[0, 1, T - 1], np.linspace(0, T - 1, 6).astype(int)]))
    _run_full("bitplane", tokens, 160, T=T)


@pytest.mark.timeout(600)
def test_int3_layer_prefill_batch_full_size_sampled():
    """The int3 Mixtral-shaped decode layer (H 4096, I 14336, G128, rank 32,
    outliers, Zipf-skewed routing) with a prefill batch of 2048 tokens
    (512 pairs per expert on average): its default path is then the tiled
    one, with the 3-bit field decode."""
    T = 2048
    tokens = np.unique(np.concatenate([[0, 1, T - 1], np.linspace(0, T - 1, 5).astype(int)]))
    _run_full("decode", tokens, 192, T=T)
