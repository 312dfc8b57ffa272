"""Runtime bitwidth of bit-plane blocks (weight pages whose committed
bitwidth changes at run time): after commits the layer's output equals the
oracle's at the new bitwidths; committing back restores the original output
bit for bit; bit-planes that no committed bitwidth reads can be paged out
(overwritten) and back without changing the output."""

import numpy as np
import pytest

from synth import configs, gen
from tests import layers

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CFG = configs.reduced(configs.get("bitplane"), E=32, T=128)


def _run(dev, x, logits, n_comp, path=0):
    from bit_quantized_moe_token_amd import moeq
    rt = moeq.route(torch.from_numpy(logits).cuda(), CFG["k"])
    y = moeq.expert_ffn(dev, torch.from_numpy(x).cuda(), rt, n_comp, out_dtype=torch.float32, path=path)
    torch.cuda.synchronize()
    return y


def _lut(e, blk, q):
    from bit_quantized_moe_token_amd import moeq
    W = torch.from_numpy(gen.gen_weight_block(CFG, 0, e, blk)).cuda()
    c, s, z = moeq.quantize_rtn(W, 4, CFG["G"])
    return moeq.build_lut(W, c, s, z, q, CFG["G"])


@pytest.fixture(scope="module")
def setup():
    orc0 = layers.oracle_layer(CFG, 0, cache_blocks=3 * CFG["E"])
    dev = layers.device_layer(CFG, 0, orc0)
    x = gen.gen_x(CFG, 0)
    logits = gen.gen_logits(CFG, 0)
    return dev, x, logits


def test_commit_changes_bitwidth(setup):
    dev, x, logits = setup
    E, n_comp = CFG["E"], CFG["n_comp"]
    bits0 = gen.gen_bits(CFG, 0)
    y0 = _run(dev, x, logits, n_comp)
    bytes0 = sum(dev.block_bytes(e, b) for e in range(E) for b in range(3))
    bits1 = (bits0 - 2 + 1) % 3 + 2                     # 2 -> 3 -> 4 -> 2 on every block
    for e in range(E):
        for b in range(3):
            dev.commit_bits(e, b, int(bits1[e, b]), _lut(e, b, int(bits1[e, b])))
            assert dev.committed_bits(e, b) == bits1[e, b]
    y1 = _run(dev, x, logits, n_comp)
    orc1 = layers.oracle_layer(CFG, 0, cache_blocks=3 * E, bits=bits1)
    ref1 = layers.oracle_y(orc1, CFG, x, logits, n_comp)
    layers.check_y(y1.cpu().numpy(), ref1, "committed bits")
    # the tiled path reads the same committed planes and tables
    layers.check_y(_run(dev, x, logits, n_comp, path=3).cpu().numpy(), ref1, "committed bits, tiled")
    # committed bytes follow the planes and tables now read
    N_K = {0: CFG["I"] * CFG["H"], 1: CFG["I"] * CFG["H"], 2: CFG["H"] * CFG["I"]}
    want = bytes0 + sum(N_K[b] * (int(bits1[e, b]) - int(bits0[e, b])) // 8 +
                        N_K[b] // 128 * (2 << int(bits1[e, b])) - N_K[b] // 128 * (2 << int(bits0[e, b]))
                        for e in range(E) for b in range(3))
    assert sum(dev.block_bytes(e, b) for e in range(E) for b in range(3)) == want
    # back to the packed bitwidths: the original output, bit for bit
    for e in range(E):
        for b in range(3):
            dev.commit_bits(e, b, int(bits0[e, b]), _lut(e, b, int(bits0[e, b])))
    assert torch.equal(_run(dev, x, logits, n_comp), y0)


def test_paged_out_planes_are_not_read(setup):
    dev, x, logits = setup
    E, n_comp = CFG["E"], CFG["n_comp"]
    bits0 = gen.gen_bits(CFG, 0)
    e, b = 3, 2
    dev.commit_bits(e, b, 2, _lut(e, b, 2))
    bits2 = bits0.copy()
    bits2[e, b] = 2
    y2 = _run(dev, x, logits, n_comp)
    base = dev.buf.data_ptr()
    saved = []
    for plane in (2, 3):                                # the two least significant planes
        ptr, n = dev.plane_region(e, b, plane)
        view = dev.buf[ptr - base:ptr - base + n]
        saved.append((view, view.cpu().clone()))        # paged out to host ...
        view.fill_(0xA5)                                # ... and the device bytes reused
    torch.cuda.synchronize()
    assert torch.equal(_run(dev, x, logits, n_comp), y2)
    orc2 = layers.oracle_layer(CFG, 0, cache_blocks=3 * E, bits=bits2)
    ref2 = layers.oracle_y(orc2, CFG, x, logits, n_comp)
    layers.check_y(y2.cpu().numpy(), ref2, "q=2 block")
    # nor does the tiled path read them
    layers.check_y(_run(dev, x, logits, n_comp, path=3).cpu().numpy(), ref2, "q=2 block, tiled")
    for view, host in saved:                            # paged back in, then committed
        view.copy_(host.cuda())
    dev.commit_bits(e, b, 4, _lut(e, b, 4))
    bits4 = bits0.copy()
    bits4[e, b] = 4
    y4 = _run(dev, x, logits, n_comp)
    orc4 = layers.oracle_layer(CFG, 0, cache_blocks=3 * E, bits=bits4)
    layers.check_y(y4.cpu().numpy(), layers.oracle_y(orc4, CFG, x, logits, n_comp), "q=4 block")
    dev.commit_bits(e, b, int(bits0[e, b]), _lut(e, b, int(bits0[e, b])))


def test_commit_rejections(setup):
    from bit_quantized_moe_token_amd import moeq
    dev, x, logits = setup
    lut = _lut(0, 0, 3)
    with pytest.raises(moeq.MoeqError):
        dev.commit_bits(0, 0, 5, lut)
    with pytest.raises(moeq.MoeqError):
        dev.commit_bits(CFG["E"], 0, 3, lut)
    tiny = configs.get("tiny")
    int_layer = layers.device_layer(tiny, 0, layers.oracle_layer(tiny, 0))
    with pytest.raises(moeq.MoeqError):
        int_layer.commit_bits(0, 0, 3, torch.zeros((tiny["I"], tiny["H"] // tiny["G"], 16),
                                                   dtype=torch.float16, device="cuda"))


def test_release_reload_cycle(setup):
    """Page movement through the library: lower eight experts' blocks to
    q = 2 and release their two low planes to pinned host memory on a side
    stream, reuse (overwrite) the freed device bytes there, reload, and
    commit q = 4 on the compute stream with no host synchronisation in
    between (the commit waits for the reload itself).  The output matches
    the oracle at every step, and committing the packed bitwidths back
    restores the first output bit for bit."""
    from bit_quantized_moe_token_amd import moeq
    dev, x, logits = setup
    E, n_comp = CFG["E"], CFG["n_comp"]
    bits0 = gen.gen_bits(CFG, 0)
    y0 = _run(dev, x, logits, n_comp)
    blocks = [(e, b) for e in range(8) for b in range(3)]
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    luts = {(e, b, q): _lut(e, b, q) for e, b in blocks for q in (2, 4)}
    torch.cuda.synchronize()
    host = {}
    base = dev.buf.data_ptr()
    for e, b in blocks:
        assert dev.resident_planes(e, b) == 4
        dev.set_desired_bits(e, b, 2)
        assert dev.desired_bits(e, b) == 2
        dev.commit_bits(e, b, 2, luts[(e, b, 2)])                   # lower first ...
        ptr, pb = dev.plane_region(e, b, 0)
        host[(e, b)] = torch.empty(4 * pb, dtype=torch.uint8, pin_memory=True)
        dev.plane_release(e, b, host[(e, b)], stream=side)           # ... then release
        assert dev.resident_planes(e, b) == 2
        with torch.cuda.stream(side):                                # reuse the freed bytes
            p2, _ = dev.plane_region(e, b, 2)
            dev.buf[p2 - base:p2 - base + 2 * pb].fill_(0xA5)
    with pytest.raises(moeq.MoeqError):                              # planes 2, 3 are gone
        dev.commit_bits(0, 0, 4, luts[(0, 0, 4)])
    bits2 = bits0.copy()
    for e, b in blocks:
        bits2[e, b] = 2
    y2 = _run(dev, x, logits, n_comp)
    orc2 = layers.oracle_layer(CFG, 0, cache_blocks=3 * E, bits=bits2)
    layers.check_y(y2.cpu().numpy(), layers.oracle_y(orc2, CFG, x, logits, n_comp), "released planes")
    for e, b in blocks:                                              # reload, then raise
        dev.set_desired_bits(e, b, 4)
        dev.plane_reload(e, b, 4, host[(e, b)], stream=side)
        assert dev.resident_planes(e, b) == 4
        dev.commit_bits(e, b, 4, luts[(e, b, 4)])                    # on `main`, after the reload
    assert torch.cuda.current_stream() == main
    bits4 = bits0.copy()
    for e, b in blocks:
        bits4[e, b] = 4
    y4 = _run(dev, x, logits, n_comp)
    orc4 = layers.oracle_layer(CFG, 0, cache_blocks=3 * E, bits=bits4)
    layers.check_y(y4.cpu().numpy(), layers.oracle_y(orc4, CFG, x, logits, n_comp), "reloaded planes")
    for e, b in blocks:
        dev.commit_bits(e, b, int(bits0[e, b]), _lut(e, b, int(bits0[e, b])))
    assert torch.equal(_run(dev, x, logits, n_comp), y0)


def test_page_movement_rejections(setup):
    from bit_quantized_moe_token_amd import moeq
    dev, x, logits = setup
    small = torch.empty(16, dtype=torch.uint8, pin_memory=True)
    dev.commit_bits(1, 1, 2, _lut(1, 1, 2))
    with pytest.raises(moeq.MoeqError):                              # host buffer too small
        dev.plane_release(1, 1, small)
    with pytest.raises(moeq.MoeqError):
        dev.set_desired_bits(1, 1, 5)
    with pytest.raises(moeq.MoeqError):
        dev.plane_reload(1, 1, 1, small)
    dev.commit_bits(1, 1, int(gen.gen_bits(CFG, 0)[1, 1]), _lut(1, 1, int(gen.gen_bits(CFG, 0)[1, 1])))
    tiny = configs.get("tiny")
    int_layer = layers.device_layer(tiny, 0, layers.oracle_layer(tiny, 0))
    with pytest.raises(moeq.MoeqError):
        int_layer.resident_planes(0, 0)
