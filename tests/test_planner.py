"""The bit-plane release planner: the library's host planner against the
oracle's greedy on random instances (same actions in the same order), the
oracle pinned by hand-worked examples, by the empty/infeasible targets and
against an exhaustive search on tiny inputs (the greedy never beats the
optimum; its gap is reported)."""

import numpy as np
import pytest

from oracle import planner


def _instance(rng, n):
    q = rng.integers(2, 5, size=n)
    plane = rng.integers(1, 9, size=n).astype(np.float64) * 1024.0       # one bit-plane, bytes
    lut = np.array([4.0, 8.0, 16.0]) * 2 * 64                            # table bytes at q = 2, 3, 4
    bytes_tbl = np.stack([plane * qq + lut[qq - 2] for qq in (2, 3, 4)], axis=1)
    g = rng.uniform(0.0, 2.0, size=(n, 3))
    mu = rng.choice([0.5, 1.0, 4.0], size=n)
    eta = np.exp(rng.normal(0, 0.3, size=n))
    return q, bytes_tbl, g, mu, eta


def test_oracle_hand_examples():
    # two blocks at q = 4; plane bytes 100 and 300 (no tables); g flat
    bytes_tbl = [[200.0, 300.0, 400.0], [600.0, 900.0, 1200.0]]
    g = [[1.0, 1.0, 1.0], [1.5, 1.5, 1.5]]
    mu, eta = [1.0, 1.0], [1.0, 1.0]
    # damage per byte: block 0 1/100, block 1 1.5/300 = 1/200 -> block 1 first
    assert planner.greedy_plan([4, 4], bytes_tbl, g, mu, eta, 0.0, 250.0) == ([4, 3], [1], 300.0, 1.5)
    assert planner.greedy_plan([4, 4], bytes_tbl, g, mu, eta, 0.0, 301.0) == ([4, 2], [1, 1], 600.0, 3.0)
    assert planner.greedy_plan([4, 4], bytes_tbl, g, mu, eta, 0.0, 601.0) == ([3, 2], [1, 1, 0], 700.0, 4.0)
    # the floor eps lifts a zero-sensitivity block's damage
    assert planner.greedy_plan([3, 3], bytes_tbl, [[0.0] * 3, [1.0] * 3], mu, eta, 2.0, 50.0) == \
        ([3, 2], [1], 300.0, 2.0)
    # no target: no action; unreachable target: everything to q = 2
    assert planner.greedy_plan([4, 3], bytes_tbl, g, mu, eta, 0.0, 0.0) == ([4, 3], [], 0.0, 0.0)
    q, order, rel, dmg = planner.greedy_plan([4, 3], bytes_tbl, g, mu, eta, 0.0, 1e9)
    assert q == [2, 2] and rel == 500.0 and len(order) == 3


@pytest.mark.parametrize("seed", range(6))
def test_greedy_within_exhaustive_optimum(seed):
    rng = np.random.default_rng(seed)
    q, bytes_tbl, g, mu, eta = _instance(rng, 4)
    total = float(sum(bytes_tbl[i][q[i] - 2] - bytes_tbl[i][0] for i in range(4)))
    for frac in (0.1, 0.4, 0.8):
        target = frac * total
        qg, order, rel, dmg = planner.greedy_plan(q, bytes_tbl, g, mu, eta, 0.01, target)
        best = planner.exact_plan(q, bytes_tbl, g, mu, eta, 0.01, target)
        if total > 0:
            assert best is not None and rel >= target
            assert dmg >= best[0] - 1e-12
            print(f"seed {seed} target {frac:.1f}: greedy {dmg:.4f} optimum {best[0]:.4f}")


@pytest.mark.parametrize("seed", range(8))
def test_library_planner_matches_oracle(seed):
    from bit_quantized_moe_token_amd import moeq
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 200))
    q, bytes_tbl, g, mu, eta = _instance(rng, n)
    total = float(sum(bytes_tbl[i][q[i] - 2] - bytes_tbl[i][0] for i in range(n)))
    for target in (0.0, 0.05 * total, 0.5 * total, 2.0 * total + 1):
        ref = planner.greedy_plan(q, bytes_tbl, g, mu, eta, 0.05, target)
        got = moeq.plan_reductions(q, bytes_tbl, g, mu, eta, 0.05, target)
        assert got[0].tolist() == ref[0] and got[1] == ref[1]
        assert got[2] == pytest.approx(ref[2], rel=1e-12) and got[3] == pytest.approx(ref[3], rel=1e-12)


def test_library_planner_validation():
    from bit_quantized_moe_token_amd import moeq
    with pytest.raises(moeq.MoeqError):
        moeq.plan_reductions([5], [[1, 2, 3]], [[1, 1, 1]], [1], [1], 0.0, 10.0)
    with pytest.raises(moeq.MoeqError):
        moeq.plan_reductions([3], [[3, 2, 1]], [[1, 1, 1]], [1], [1], 0.0, 10.0)
