"""GPU parity of the routed expert layer against the fp64 oracle on the five
seeded workloads (reduced dimensions where the oracle would be slow, with
the same structure), plus compensation switches, determinism and token
permutation."""

import numpy as np
import pytest

from synth import configs, gen
from tests import layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# (config, overrides) — reduced Mixtral layers keep H, I multiples of 128
# with a ragged tile tail (1792 / 128 = 14 tiles); T keeps the regime
CASES = {
    "tiny": ("tiny", {}),
    "decode": ("decode", dict(H=512, I=1792)),
    # int4, T = 1536, k = 2, E = 8: 384 pairs per expert on average
    "prefill": ("prefill", dict(H=512, I=1792, T=1536)),
    # the int3 layer with as many tokens (where its default turns tiled)
    "decode_many": ("decode", dict(H=512, I=1792, T=1536)),
    # many pairs and I >= 4096: the down projection runs in wave tiles
    # (each wave a 16-pair tile of a 64-pair chunk, K split over the grid)
    "prefill_wide": ("prefill", dict(H=512, I=4096, T=1024)),
    "finegrained": ("finegrained", {}),
    "bitplane": ("bitplane", dict(E=32, T=128)),
    # the largest expert count (256): experts with one or two pairs, chunk
    # lookup over four 64-lane passes, routing with E = 256
    "many_experts": ("finegrained", dict(E=256, k=8, T=48, H=256, I=256)),
    "many_experts_bitplane": ("bitplane", dict(E=256, T=40, H=256, I=256)),
    # bit-plane blocks with many tokens per expert (256 pairs on average:
    # full and partial 128-token tiles), a ragged last group of K tiles in
    # the down projection (I = 768: 6 tiles)
    "bitplane_wide": ("bitplane", dict(E=16, T=512, H=512, I=768)),
    # shared factors on an INT layer (groups of 4 of 16 experts, so a
    # token's six experts often share groups) whose low-rank terms are a
    # large part of the output (factors N(0, 0.05)); two of six slots
    # compensated, so the groups' leaders come from those slots only
    "shared_int": ("finegrained", dict(E=16, T=64, H=512, I=1408, rs=32, share=4, factor_std=0.05)),
}

_cache = {}


def _setup(case, seed=0):
    key = (case, seed)
    if key not in _cache:
        name, over = CASES[case]
        cfg = configs.reduced(configs.get(name), **over) if over else configs.get(name)
        orc = layers.oracle_layer(cfg, seed, cache_blocks=3 * cfg["E"])
        dev = layers.device_layer(cfg, seed, orc)
        x = gen.gen_x(cfg, seed)
        logits = gen.gen_logits(cfg, seed)
        _cache.clear()
        _cache[key] = (cfg, orc, dev, x, logits)
    return _cache[key]


PATH_AUTO, PATH_STREAM, PATH_TILED = 0, 1, 3


def _run(dev, cfg, x, logits, n_comp, out_dtype=torch.float16, split_k=0, path=PATH_AUTO):
    from bit_quantized_moe_token_amd import moeq
    xd = torch.from_numpy(x).cuda()
    rt = moeq.route(torch.from_numpy(logits).cuda(), cfg["k"])
    y = moeq.expert_ffn(dev, xd, rt, n_comp, out_dtype=out_dtype, split_k=split_k, path=path)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", list(CASES))
def test_ffn_matches_oracle(case, seed):
    cfg, orc, dev, x, logits = _setup(case, seed)
    y = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32)
    ref = layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"])
    rel, fro = layers.check_y(y.cpu().numpy(), ref, case)
    print(f"{case} seed {seed}: max|err|/rms {rel:.2e}  fro {fro:.2e}")
    # fp16 output stays inside the same bound
    y16 = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float16)
    layers.check_y(y16.float().cpu().numpy(), ref, f"{case} seed {seed} fp16")


@pytest.mark.parametrize("case", ["tiny", "finegrained", "bitplane", "shared_int", "prefill_wide"])
def test_ffn_compensation_switch(case):
    """n_comp in {0, 1, k} against the oracle; n_comp = 0 equals the layer
    without factors bit for bit."""
    cfg, orc, dev, x, logits = _setup(case)
    k = cfg["k"]
    for n_comp in (0, 1, k):
        y = _run(dev, cfg, x, logits, n_comp, out_dtype=torch.float32)
        layers.check_y(y.cpu().numpy(), layers.oracle_y(orc, cfg, x, logits, n_comp), f"{case} n_comp={n_comp}")


@pytest.mark.parametrize("case,path", [("decode", PATH_STREAM), ("prefill", PATH_STREAM),
                                       ("prefill", PATH_TILED), ("finegrained", PATH_AUTO),
                                       ("prefill_wide", PATH_TILED), ("prefill_wide", PATH_STREAM)])
def test_ffn_expert_reached_only_by_uncompensated_slots(case, path):
    """Router-guided top-n compensation with n_comp = 1 when one expert is
    every token's second choice: all of its pairs are uncompensated, so its
    tiles skip the low-rank projections (zero z rows, no V loads; the down
    projection still stores their renormalised h).  Parity with the oracle,
    on few pairs (one 16-pair tile per workgroup) and on many (a 64-pair
    chunk per workgroup), streaming and tiled."""
    from bit_quantized_moe_token_amd import moeq
    cfg, orc, dev, x, logits = _setup(case)
    assert cfg["k"] >= 2
    lg = logits.copy()
    e2 = cfg["E"] - 1
    others = np.sort(np.delete(lg, e2, axis=1), axis=1)
    lg[:, e2] = ((others[:, -1].astype(np.float64) + others[:, -2]) / 2).astype(np.float32)
    rt = moeq.route(torch.from_numpy(lg).cuda(), cfg["k"])
    ids = rt.ids.cpu().numpy()
    assert (ids[:, 1] == e2).all() and (ids[:, 0] != e2).all()
    y = _run(dev, cfg, x, lg, 1, out_dtype=torch.float32, path=path)
    layers.check_y(y.cpu().numpy(), layers.oracle_y(orc, cfg, x, lg, 1), f"{case} second-choice expert n_comp=1")


def test_rank0_bitwise_equals_uncompensated():
    from bit_quantized_moe_token_amd import moeq
    cfg, orc, dev, x, logits = _setup("tiny")
    y0 = _run(dev, cfg, x, logits, 0, out_dtype=torch.float32)
    # the same codes packed without any factors
    E = cfg["E"]
    bits = gen.gen_bits(cfg, 0)
    blocks = [moeq.quantize_block(torch.from_numpy(gen.gen_weight_block(cfg, 0, e, b)).cuda(),
                                  "int", int(bits[e, b]), cfg["G"]) for e in range(E) for b in range(3)]
    plain = moeq.PackedLayer(E, cfg["H"], cfg["I"], cfg["G"], "int", bits, blocks)
    y1 = _run(plain, cfg, x, logits, cfg["k"], out_dtype=torch.float32)
    assert torch.equal(y0, y1)


def test_ffn_wave_tiles_uneven_k_split():
    """Wave tiles whose K split does not divide the 32-column steps evenly
    (I = 8320: 260 steps over 8 grid slices), on both paths, against the
    oracle; and bit-identical on a repeat (fixed order of the partials)."""
    cfg = configs.reduced(configs.get("prefill"), H=256, I=8320, T=1024)
    orc = layers.oracle_layer(cfg, 0, cache_blocks=3 * cfg["E"])
    dev = layers.device_layer(cfg, 0, orc)
    x, logits = gen.gen_x(cfg, 0), gen.gen_logits(cfg, 0)
    ref = layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"])
    for path in (PATH_TILED, PATH_STREAM):
        y = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, path=path)
        layers.check_y(y.cpu().numpy(), ref, f"I=8320 path {path}")
        assert torch.equal(y, _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, path=path))


@pytest.mark.parametrize("case", ["decode", "finegrained"])
def test_ffn_deterministic_and_split_invariant(case):
    cfg, orc, dev, x, logits = _setup(case)
    a = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32)
    b = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32)
    assert torch.equal(a, b)
    ref = layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"])
    for s in (1, 2, 3, 6):     # 6: more splits than the combine requests up front
        c = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, split_k=s)
        layers.check_y(c.cpu().numpy(), ref, f"{case} split_k={s}")


@pytest.mark.parametrize("case", ["tiny", "finegrained"])
def test_ffn_token_permutation(case):
    """Permuting tokens (and their logits) permutes the output exactly."""
    cfg, orc, dev, x, logits = _setup(case)
    perm = np.random.default_rng(5).permutation(cfg["T"])
    y = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32)
    yp = _run(dev, cfg, x[perm].copy(), logits[perm].copy(), cfg["n_comp"], out_dtype=torch.float32)
    assert torch.equal(yp, y[torch.from_numpy(perm).cuda()])


def test_ffn_zero_input_and_few_tokens():
    cfg, orc, dev, x, logits = _setup("tiny")
    y = _run(dev, cfg, np.zeros_like(x), logits, cfg["k"], out_dtype=torch.float32)
    assert torch.count_nonzero(y) == 0
    for T in (1, 3, 17):
        sub = dict(cfg, T=T)
        y = _run(dev, sub, x[:T].copy(), logits[:T].copy(), cfg["k"], out_dtype=torch.float32)
        layers.check_y(y.cpu().numpy(), layers.oracle_y(orc, sub, x[:T], logits[:T], cfg["k"]), f"T={T}")


# ---- tiled path (many tokens per expert): forced on every workload,
# including one token tile per expert (decode), mixed 2/3/4-bit blocks with
# group 64 and an odd, ragged K-tile count (fine-grained: I = 1408 = 11
# tiles), and bit-plane blocks at mixed committed q with shared factors
# (one or two pairs per expert, and 256)

@pytest.mark.parametrize("case", ["tiny", "decode", "prefill", "finegrained", "shared_int", "bitplane",
                                  "many_experts_bitplane", "bitplane_wide"])
def test_ffn_tiled_path_matches_oracle(case):
    cfg, orc, dev, x, logits = _setup(case)
    ref = layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"])
    y = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, path=PATH_TILED)
    rel, fro = layers.check_y(y.cpu().numpy(), ref, case + " tiled")
    print(f"{case} tiled: max|err|/rms {rel:.2e}  fro {fro:.2e}")
    y0 = _run(dev, cfg, x, logits, 0, out_dtype=torch.float32, path=PATH_TILED)
    layers.check_y(y0.cpu().numpy(), layers.oracle_y(orc, cfg, x, logits, 0), case + " tiled n_comp=0")


def test_ffn_prefill_paths():
    """For an int4 layer the default path is the tiled one from an average
    of 96 pairs per expert (this batch) and the streaming one below (its
    first 256 tokens, 64 pairs per expert); each path gives the oracle's
    result within the tolerance."""
    cfg, orc, dev, x, logits = _setup("prefill")
    assert cfg["fmt"] == "int" and cfg["bits"] == 4 and cfg["T"] * cfg["k"] >= 96 * cfg["E"]
    ref = layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"])
    auto = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32)
    tiled = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, path=PATH_TILED)
    assert torch.equal(auto, tiled)
    stream = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, path=PATH_STREAM)
    layers.check_y(stream.cpu().numpy(), ref, "prefill stream")
    small = dict(cfg, T=256)
    xs, ls = x[:256].copy(), logits[:256].copy()
    auto_s = _run(dev, small, xs, ls, cfg["n_comp"], out_dtype=torch.float32)
    stream_s = _run(dev, small, xs, ls, cfg["n_comp"], out_dtype=torch.float32, path=PATH_STREAM)
    assert torch.equal(auto_s, stream_s)
    layers.check_y(auto_s.cpu().numpy(), layers.oracle_y(orc, small, xs, ls, cfg["n_comp"]), "prefill T=256 auto")
    perm = np.random.default_rng(7).permutation(cfg["T"])
    tp = _run(dev, cfg, x[perm].copy(), logits[perm].copy(), cfg["n_comp"], out_dtype=torch.float32,
              path=PATH_TILED)
    assert torch.equal(tp, tiled[torch.from_numpy(perm).cuda()])


def test_ffn_default_path_int3():
    """A layer with 3-bit blocks takes the tiled path only from an average of
    384 pairs per expert (this batch); at 256 (its first 1024 tokens) it
    streams."""
    cfg, orc, dev, x, logits = _setup("decode_many")
    assert cfg["bits"] == 3 and cfg["T"] * cfg["k"] == 384 * cfg["E"]
    auto = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32)
    tiled = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, path=PATH_TILED)
    assert torch.equal(auto, tiled)
    layers.check_y(auto.cpu().numpy(), layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"]), "int3 T=1536 auto")
    small = dict(cfg, T=1024)
    xs, ls = x[:1024].copy(), logits[:1024].copy()
    auto_s = _run(dev, small, xs, ls, cfg["n_comp"], out_dtype=torch.float32)
    stream_s = _run(dev, small, xs, ls, cfg["n_comp"], out_dtype=torch.float32, path=PATH_STREAM)
    assert torch.equal(auto_s, stream_s)


def _gateup_kernel_run(dev, cfg, x, logits):
    """Name of the gate/up kernel the default path launches."""
    from bit_quantized_moe_token_amd import moeq
    moeq.profile_enable(True)
    try:
        _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32)
        names = set(moeq.profile_read())
    finally:
        moeq.profile_enable(False)
    gu = sorted(n for n in names if n.startswith("gateup"))
    assert len(gu) == 1, names
    return gu[0]


def test_default_path_boundary():
    """The default path turns tiled at an average of exactly 96 pairs per
    expert on an int4 layer whose tiled grid is large enough (E = 8, k = 2,
    I = 3584: T = 384 tiles, T = 380 streams), and a layer whose tiled grid
    would leave most CUs idle (H = 256, I = 512, 124 workgroups at 384 pairs
    per expert) streams at any batch."""
    cfg = configs.reduced(configs.get("prefill"), H=512, I=3584, T=384)
    dev = layers.device_layer(cfg, 0)
    x, logits = gen.gen_x(cfg, 0), gen.gen_logits(cfg, 0)
    assert cfg["T"] * cfg["k"] == 96 * cfg["E"]
    assert _gateup_kernel_run(dev, cfg, x, logits) == "gateup_tiled"
    c95 = dict(cfg, T=380)
    assert _gateup_kernel_run(dev, c95, x[:380].copy(), logits[:380].copy()) == "gateup_stream"
    del dev
    tiny = configs.reduced(configs.get("tiny"), T=1536)
    dev = layers.device_layer(tiny, 0, layers.oracle_layer(tiny, 0, cache_blocks=3 * tiny["E"]))
    assert _gateup_kernel_run(dev, tiny, gen.gen_x(tiny, 0), gen.gen_logits(tiny, 0)) == "gateup_stream"


def test_default_path_boundary_bitplane():
    """A bit-plane layer takes the tiled path from an average of 192 pairs
    per expert (E = 16, k = 8, I = 1536: T = 384; its tiled grid has 468
    workgroups) and streams at 188 (T = 376)."""
    cfg = configs.reduced(configs.get("bitplane"), E=16, T=384, H=512, I=1536)
    dev = layers.device_layer(cfg, 0)
    x, logits = gen.gen_x(cfg, 0), gen.gen_logits(cfg, 0)
    assert cfg["T"] * cfg["k"] == 192 * cfg["E"]
    assert _gateup_kernel_run(dev, cfg, x, logits) == "gateup_tiled"
    c188 = dict(cfg, T=376)
    assert _gateup_kernel_run(dev, c188, x[:376].copy(), logits[:376].copy()) == "gateup_stream"


def test_ffn_tiled_bitplane_deterministic_and_permutation():
    """The tiled bit-plane path is bit-identical on a repeat and under a
    permutation of the tokens (each token's output is its own sum in slot
    order, whatever tile its pairs land in)."""
    cfg, orc, dev, x, logits = _setup("bitplane_wide")
    y = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, path=PATH_TILED)
    assert torch.equal(y, _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32, path=PATH_TILED))
    perm = np.random.default_rng(11).permutation(cfg["T"])
    yp = _run(dev, cfg, x[perm].copy(), logits[perm].copy(), cfg["n_comp"], out_dtype=torch.float32,
              path=PATH_TILED)
    assert torch.equal(yp, y[torch.from_numpy(perm).cuda()])


def test_ffn_tiled_rejects_unsupported_shape():
    """The tiled kernels need H to be a multiple of 256 (two-strip output
    tiles of the down projection); a forced tiled call on H = 384 is
    rejected before anything runs, and the default path streams."""
    from bit_quantized_moe_token_amd import moeq
    cfg = configs.reduced(configs.get("tiny"), H=384, T=16)
    orc = layers.oracle_layer(cfg, 0, cache_blocks=3 * cfg["E"])
    dev = layers.device_layer(cfg, 0, orc)
    x, logits = gen.gen_x(cfg, 0), gen.gen_logits(cfg, 0)
    with pytest.raises(moeq.MoeqError):
        _run(dev, cfg, x, logits, cfg["n_comp"], path=PATH_TILED)
    y = _run(dev, cfg, x, logits, cfg["n_comp"], out_dtype=torch.float32)
    layers.check_y(y.cpu().numpy(), layers.oracle_y(orc, cfg, x, logits, cfg["n_comp"]), "H=384 default")
