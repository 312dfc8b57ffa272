"""Pins of the oracle's encoding step (RTN codes, bit-plane LUTs, SVD
compensators) against hand-derived examples, invariants and closed forms."""

import json
import os

import numpy as np
import pytest

from oracle import forward, ptq

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("rtn_worked_examples.json")["cases"], ids=lambda c: c["name"])
def test_rtn_worked_examples(case):
    W = np.array([case["w"]], dtype=np.float16)
    codes, s16, z = ptq.rtn_quantize(W, case["b"], 4)
    assert codes[0].tolist() == case["codes"]
    assert float(s16[0, 0]) == case["s16"]
    assert int(z[0, 0]) == case["z"]
    w_hat = forward.dequant_int(codes, s16, z, 4)[0]
    assert w_hat.tolist() == case["w_hat"]


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("G", [64, 128])
def test_rtn_error_bound_and_ranges(b, G):
    """|w - w_hat| <= s16/2 + (2^b-1)|s - s16| in every group; z, c in range."""
    rng = np.random.default_rng(1234 + b + G)
    W = (rng.standard_normal((64, 4 * G)) * 0.02).astype(np.float16)
    W[3, :G] = 0.0                                  # a degenerate group
    W[5, G:2 * G] = np.abs(W[5, G:2 * G])           # all-positive group
    codes, s16, z = ptq.rtn_quantize(W, b, G)
    qmax = 2 ** b - 1
    assert codes.max() <= qmax and z.max() <= qmax
    w_hat = forward.dequant_int(codes, s16, z, G)
    Wd = W.astype(np.float64).reshape(64, 4, G)
    lo = np.minimum(0, Wd.min(-1))
    hi = np.maximum(0, Wd.max(-1))
    s = (hi - lo) / qmax
    sd = s16.astype(np.float64)
    bound = sd / 2 + qmax * np.abs(s - sd)
    err = np.abs(W.astype(np.float64) - w_hat).reshape(64, 4, G).max(-1)
    ok = (hi != lo)
    assert np.all(err[ok] <= bound[ok] * (1 + 1e-12))
    assert np.all(err[~ok] == 0) and np.all(sd[~ok] == 1.0)


def test_dequant_hand_enumerated():
    """INT dequant: w_hat = s (c - z), enumerated by hand for every code."""
    cases = [
        (2, 0.25, 1, [-0.25, 0.0, 0.25, 0.5]),
        (3, 0.125, 3, [-0.375, -0.25, -0.125, 0.0, 0.125, 0.25, 0.375, 0.5]),
        (4, 0.0625, 8, [(c - 8) / 16 for c in range(16)]),
    ]
    for b, s, z, expect in cases:
        n = 2 ** b
        codes = np.arange(n, dtype=np.uint8)[None, :]
        s16 = np.full((1, 1), s, dtype=np.float16)
        zz = np.full((1, 1), z, dtype=np.uint8)
        got = forward.dequant_int(codes, s16, zz, n)[0]
        assert got.tolist() == expect


def test_bitplane_index_and_lookup():
    gold = _load("bitplane_lut_examples.json")
    for c in gold["index_cases"]:
        assert int(ptq.bitplane_index(np.array([c["c4"]]), c["q"])[0]) == c["index"]
        lut = np.zeros((1, 1, 16), dtype=np.float16)
        lut[0, 0, :] = 100 + np.arange(16)
        got = forward.dequant_bitplane(np.array([[c["c4"]]], dtype=np.uint8), lut, c["q"], 1)
        assert got[0, 0] == c["lut_100_plus_j"]


def test_bitplane_lut_worked_examples():
    gold = _load("bitplane_lut_examples.json")
    for c in gold["lut_cases"]:
        W = np.array([c["w"]], dtype=np.float16)
        c4, s16, z = ptq.rtn_quantize(W, 4, 4)
        assert c4[0].tolist() == c["c4"]
        assert float(s16[0, 0]) == c["s16"] and int(z[0, 0]) == c["z"]
        lut = ptq.bitplane_lut(W, c4, s16, z, c["q"], 4)[0, 0]
        if "lut" in c:
            assert lut[:len(c["lut"])].astype(float).tolist() == c["lut"]
            assert np.all(lut[len(c["lut"]):] == 0)
        for j, v in c.get("lut_slots", {}).items():
            assert float(lut[int(j)]) == v


def test_bitplane_q4_with_affine_lut_equals_int4():
    """Cross-format identity: LUT[j] = s16 (j - z) at q = 4 gives the INT b=4
    dequantization bit for bit (scales are powers of two so the LUT entries
    are exact in fp16)."""
    rng = np.random.default_rng(3)
    c4 = rng.integers(0, 16, size=(32, 256)).astype(np.uint8)
    s16 = (2.0 ** rng.integers(-12, -2, size=(32, 2))).astype(np.float16)
    z = rng.integers(0, 16, size=(32, 2)).astype(np.uint8)
    vals = s16.astype(np.float64)[..., None] * (np.arange(16)[None, None, :] - z.astype(np.float64)[..., None])
    lut = vals.astype(np.float16)
    assert np.array_equal(lut.astype(np.float64), vals)
    a = forward.dequant_bitplane(c4, lut, 4, 128)
    b = forward.dequant_int(c4, s16, z, 128)
    assert np.array_equal(a, b)


def test_bitplane_lut_is_bucket_mean():
    """Each LUT slot is the fp16 mean of its bucket (brute force per group)."""
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((4, 256)) * 0.02).astype(np.float16)
    c4, s16, z = ptq.rtn_quantize(W, 4, 128)
    for q in (2, 3, 4):
        lut = ptq.bitplane_lut(W, c4, s16, z, q, 128)
        for n in range(4):
            for g in range(2):
                w = [float(v) for v in W[n, g * 128:(g + 1) * 128]]
                idx = [int(c) >> (4 - q) for c in c4[n, g * 128:(g + 1) * 128]]
                for j in range(2 ** q):
                    mem = [wv for wv, i in zip(w, idx) if i == j]
                    if mem:
                        assert lut[n, g, j] == np.float16(sum(mem) / len(mem))
                    else:
                        span = 2 ** (4 - q)
                        mid = j * span + (span - 1) / 2
                        assert lut[n, g, j] == np.float16(float(s16[n, g]) * (mid - int(z[n, g])))
                assert np.all(lut[n, g, 2 ** q:] == 0)


def test_bitplane_lut_error_shrinks_with_q():
    """More committed planes never increase the group's squared error on
    average (finer buckets of the same parent codes)."""
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((64, 512)) * 0.02).astype(np.float16)
    c4, s16, z = ptq.rtn_quantize(W, 4, 128)
    errs = []
    for q in (2, 3, 4):
        lut = ptq.bitplane_lut(W, c4, s16, z, q, 128)
        errs.append(np.sum((forward.dequant_bitplane(c4, lut, q, 128) - W.astype(np.float64)) ** 2))
    assert errs[0] > errs[1] > errs[2]


def test_svd_compensator_eckart_young():
    """||R - U V||_F^2 equals the sum of the discarded squared singular values,
    taken here from the eigenvalues of R^T R (a different routine), and the
    fp16-rounded factors still strictly reduce ||W - W_hat||_F."""
    rng = np.random.default_rng(0)
    W = (rng.standard_normal((512, 256)) * 0.02).astype(np.float16)
    codes, s16, z = ptq.rtn_quantize(W, 4, 64)
    W_hat = forward.dequant_int(codes, s16, z, 64)
    R = W.astype(np.float64) - W_hat
    ev = np.sort(np.linalg.eigvalsh(R.T @ R))[::-1]
    for r in (1, 16, 64):
        U16, V16, U64, V64, _ = ptq.svd_compensator(W, W_hat, r)
        assert U16.shape == (512, r) and V16.shape == (r, 256)
        res = np.sum((R - U64 @ V64) ** 2)
        assert res == pytest.approx(np.sum(ev[r:]), rel=1e-9)
        assert np.linalg.matrix_rank(U64 @ V64) == r
        res16 = np.sum((R - U16.astype(np.float64) @ V16.astype(np.float64)) ** 2)
        assert res16 < np.sum(R ** 2)
        # optimality: random rank-r factors never beat the truncated SVD
        for _ in range(3):
            A = rng.standard_normal((512, r))
            B = np.linalg.lstsq(A, R, rcond=None)[0]
            assert np.sum((R - A @ B) ** 2) >= res * (1 - 1e-12)
    # the balanced split puts the same singular values on both sides
    U16, V16, U64, V64, S = ptq.svd_compensator(W, W_hat, 8)
    assert np.allclose(np.linalg.norm(U64, axis=0), np.linalg.norm(V64, axis=1))


def test_mean_residual_compensator_minimizes_the_group_objective():
    """The shared pair of n residuals: the identity sum ||R_m - X||^2 =
    sum ||R_m - mean||^2 + n ||mean - X||^2 holds for it, no rank-r
    competitor (least-squares fits to random column spaces, and each
    block's own truncated SVD) gives a smaller group objective, and n = 1
    reduces to svd_compensator."""
    rng = np.random.default_rng(3)
    N, K, r, n = 96, 80, 6, 3
    common = rng.standard_normal((N, r)) @ rng.standard_normal((r, K)) * 0.01
    Ws = [(common + rng.standard_normal((N, K)) * 0.004).astype(np.float16) for _ in range(n)]
    Whs = [np.zeros((N, K)) for _ in range(n)]
    U16, V16, U64, V64, S = ptq.mean_residual_compensator(Ws, Whs, r)
    Rm = [W.astype(np.float64) for W in Ws]
    mean = sum(Rm) / n
    X = U64 @ V64
    obj = sum(np.sum((R - X) ** 2) for R in Rm)
    assert obj == pytest.approx(sum(np.sum((R - mean) ** 2) for R in Rm) + n * np.sum((mean - X) ** 2), rel=1e-12)
    assert np.linalg.matrix_rank(X) == r
    competitors = []
    for _ in range(4):
        A = rng.standard_normal((N, r))
        competitors.append(A @ np.linalg.lstsq(A, mean, rcond=None)[0])
    for R in Rm:
        _, _, Ua, Va, _ = ptq.svd_compensator(R, np.zeros_like(R), r)
        competitors.append(Ua @ Va)
    for C in competitors:
        assert sum(np.sum((R - C) ** 2) for R in Rm) >= obj * (1 - 1e-12)
    # one block: the same factors as svd_compensator
    _, _, U1, V1, _ = ptq.mean_residual_compensator(Ws[:1], Whs[:1], r)
    _, _, U2, V2, _ = ptq.svd_compensator(Ws[0], Whs[0], r)
    assert np.allclose(U1 @ V1, U2 @ V2, rtol=0, atol=1e-15)
