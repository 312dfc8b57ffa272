"""GPU parity of the encoding step and the packed layout: RTN codes, scales
and zeros and bit-plane LUTs bit-exact against the oracle's PTQ; packed
codes read back with the expert kernels' own decode bit-exact."""

import numpy as np
import pytest

from oracle import ptq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _moeq():
    from bit_quantized_moe_token_amd import moeq
    return moeq


def _weights(rng, N, K, scale=0.02):
    W = (rng.standard_normal((N, K)) * scale).astype(np.float16)
    # edge cases: an all-zero group, an all-positive group, subnormal-range
    # values, exact half-way ties on a power-of-two grid, large outliers
    G0 = min(64, K)
    W[0, :G0] = 0
    W[1, :G0] = np.abs(W[1, :G0])
    W[2, :G0] = (rng.standard_normal(G0) * 1e-6).astype(np.float16)
    W[3, :G0] = (np.arange(G0) % 7 - 3).astype(np.float16) * np.float16(0.125)
    if N > 4:
        W[4, :G0] *= np.float16(50)
    return W


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("G", [64, 128])
def test_quantize_rtn_bitexact(bits, G):
    moeq = _moeq()
    rng = np.random.default_rng(100 + bits * 10 + G)
    W = _weights(rng, 96, 640)
    c, s, z = moeq.quantize_rtn(torch.from_numpy(W).cuda(), bits, G)
    oc, os_, oz = ptq.rtn_quantize(W, bits, G)
    assert np.array_equal(c.cpu().numpy(), oc)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(z.cpu().numpy(), oz)


def test_quantize_rtn_golden_and_small_groups():
    """Hand-worked examples (tests/golden) through the device quantizer."""
    import json
    import os
    moeq = _moeq()
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rtn_worked_examples.json")))
    for case in gold["cases"]:
        W = np.array([case["w"]], dtype=np.float16)
        c, s, z = moeq.quantize_rtn(torch.from_numpy(W).cuda(), case["b"], 4)
        assert c.cpu().numpy()[0].tolist() == case["codes"], case["name"]
        assert float(s.cpu().numpy()[0, 0]) == case["s16"], case["name"]
        assert int(z.cpu().numpy()[0, 0]) == case["z"], case["name"]


@pytest.mark.parametrize("q", [2, 3, 4])
def test_build_lut_bitexact(q):
    moeq = _moeq()
    rng = np.random.default_rng(7 + q)
    W = _weights(rng, 64, 512)
    Wd = torch.from_numpy(W).cuda()
    c4, s, z = moeq.quantize_rtn(Wd, 4, 128)
    lut = moeq.build_lut(Wd, c4, s, z, q, 128)
    oc, os_, oz = ptq.rtn_quantize(W, 4, 128)
    olut = ptq.bitplane_lut(W, oc, os_, oz, q, 128)
    assert np.array_equal(lut.cpu().numpy().view(np.uint16), olut.view(np.uint16))


def _pack_single(moeq, fmt, bits, G, H, I, rng):
    """A one-expert layer whose three blocks hold random codes."""
    blocks = []
    ref = []
    for blk in range(3):
        N, K = (I, H) if blk < 2 else (H, I)
        if fmt == "int":
            c = rng.integers(0, 2 ** bits, size=(N, K)).astype(np.uint8)
            s = (rng.standard_normal((N, K // G)) * 0.01).astype(np.float16)
            z = rng.integers(0, 2 ** bits, size=(N, K // G)).astype(np.uint8)
            blocks.append(dict(codes=torch.from_numpy(c).cuda(), scales=torch.from_numpy(s).cuda(),
                               zeros=torch.from_numpy(z).cuda()))
            ref.append(c)
        else:
            c = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
            lut = (rng.standard_normal((N, K // G, 16)) * 0.01).astype(np.float16)
            blocks.append(dict(codes=torch.from_numpy(c).cuda(), lut=torch.from_numpy(lut).cuda()))
            ref.append(ptq.bitplane_index(c, bits))
    layer = moeq.PackedLayer(1, H, I, G, fmt, np.full((1, 3), bits), blocks)
    return layer, ref


@pytest.mark.parametrize("fmt,bits,G", [("int", 2, 64), ("int", 3, 64), ("int", 4, 64),
                                        ("int", 2, 128), ("int", 3, 128), ("int", 4, 128),
                                        ("bitplane", 2, 128), ("bitplane", 3, 128), ("bitplane", 4, 128)])
@pytest.mark.parametrize("H,I", [(256, 640), (512, 1408)])
def test_pack_debug_unpack_roundtrip(fmt, bits, G, H, I):
    """K/128 = 2, 4, 5 and 11 tiles: full tile groups and ragged tails."""
    moeq = _moeq()
    rng = np.random.default_rng(bits * 1000 + H + I)
    layer, ref = _pack_single(moeq, fmt, bits, G, H, I, rng)
    for blk in range(3):
        got = layer.debug_unpack(0, blk).cpu().numpy()
        assert np.array_equal(got, ref[blk]), f"block {blk}"


def test_block_bytes_accounting():
    moeq = _moeq()
    rng = np.random.default_rng(3)
    layer, _ = _pack_single(moeq, "int", 3, 128, 256, 640, rng)
    # gate: 640 x 256 weights at 3 bits + 3 bytes per 128-group
    assert layer.block_bytes(0, 0) == 640 * 256 * 3 // 8 + 640 * 2 * 3
    layer, _ = _pack_single(moeq, "bitplane", 2, 128, 256, 640, rng)
    assert layer.block_bytes(0, 2) == 256 * 640 * 2 // 8 + 256 * 5 * 4 * 2
