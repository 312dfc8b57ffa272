"""Pins of the oracle's forward pass: routing against brute force and closed
forms, the counting sort against a library stable sort, and the expert FFN /
combine against a dense-mask brute force, invariants and a hand-derived toy."""

import json
import math
import os

import numpy as np
import pytest

from oracle import forward, ptq
from oracle.layer import OracleLayer

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ routing

def _brute_topk(l, k):
    out = []
    for row in l:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(order[:k])
    return np.array(out)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (128, 8), (5, 5), (3, 1)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    # few distinct values -> many ties, which must go to the lower expert id
    l = rng.integers(-3, 4, size=(200, E)).astype(np.float32) * np.float32(0.5)
    assert np.array_equal(forward.topk_ids(l, k), _brute_topk(l, k))
    l2 = rng.standard_normal((200, E)).astype(np.float32)
    assert np.array_equal(forward.topk_ids(l2, k), _brute_topk(l2, k))


def test_gates_closed_forms():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((50, 8)).astype(np.float32)
    rt = forward.route(l, 2)
    assert np.allclose(rt["gates"].sum(1), 1.0, atol=1e-15, rtol=0)
    # top-2 gates are a logistic function of the logit gap
    sel = np.take_along_axis(l.astype(np.float64), rt["ids"].astype(np.int64), 1)
    g0 = [1.0 / (1.0 + math.exp(float(b - a))) for a, b in sel]
    assert np.allclose(rt["gates"][:, 0], g0, rtol=0, atol=1e-15)
    # k = E: the gates are the full softmax in expert-id order
    rt = forward.route(l, 8)
    for t in range(50):
        z = sum(math.exp(float(v)) for v in l[t])
        full = [math.exp(float(v)) / z for v in l[t]]
        got = np.zeros(8)
        got[rt["ids"][t]] = rt["gates"][t]
        assert np.allclose(got, full, rtol=1e-13, atol=0)
    # k = 1: one gate equal to 1
    assert np.all(forward.route(l, 1)["gates"] == 1.0)
    # gates are ordered like the logits
    rt = forward.route(l, 4)
    assert np.all(np.diff(rt["gates"], axis=1) <= 0)


@pytest.mark.parametrize("E,P", [(8, 128), (64, 1536), (128, 4096), (4, 0), (3, 1)])
def test_counting_sort_matches_stable_argsort(E, P):
    rng = np.random.default_rng(P + E)
    ids = rng.integers(0, E, size=P)
    offsets, sp, pos = forward.counting_sort(ids, E)
    ref = np.argsort(ids, kind="stable")
    assert np.array_equal(sp, ref)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(ids, minlength=E))]))
    assert offsets[-1] == P
    if P:
        assert np.array_equal(pos[sp], np.arange(P))
        assert np.all(np.diff(ids[sp]) >= 0)


def test_routing_mass_pins():
    """Routing mass: brute-force per-expert sums of the gates; k = E gives
    the full softmax column sums; the masses of all experts add up to T
    (every token's gates sum to 1); bucket edges by counting."""
    rng = np.random.default_rng(11)
    T, E = 37, 6
    logits = rng.standard_normal((T, E)).astype(np.float32)
    for k in (1, 2, E):
        rt = forward.route(logits, k)
        m = forward.routing_mass(rt["ids"], rt["gates"], E)
        brute = np.array([sum(rt["gates"][t, j] for t in range(T) for j in range(k) if rt["ids"][t, j] == e)
                          for e in range(E)])
        assert np.allclose(m, brute, rtol=0, atol=1e-12)
        assert abs(m.sum() - T) < 1e-12
        if k == E:
            l = logits.astype(np.float64)
            p = np.exp(l - l.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            assert np.allclose(m, p.sum(0), rtol=0, atol=1e-12)
    # k = 1 mass is the count of tokens whose top expert is e
    rt = forward.route(logits, 1)
    assert np.array_equal(forward.routing_mass(rt["ids"], rt["gates"], E),
                          np.bincount(rt["ids"][:, 0], minlength=E).astype(np.float64))
    edges = [1.0, 4.0, 9.5]
    assert forward.mass_bucket([0.0, 0.99, 1.0, 3.9, 4.0, 9.5, 100.0], edges).tolist() == [0, 0, 1, 1, 2, 3, 3]
    assert forward.mass_bucket([5.0], []).tolist() == [0]


# ------------------------------------------------------------------ toy layers

class _DictLayer:
    """Minimal layer over explicit quantized blocks (for the oracle pins)."""

    def __init__(self, E, H, I, G, blocks, factors=None, shared=None, share=0):
        self.E, self.H, self.I, self.G = E, H, I, G
        self._b, self._f, self._s, self.share = blocks, factors or {}, shared or {}, share

    def group_of(self, e):
        return e // self.share if self.share else 0

    def qblock(self, e, blk, rows=None):
        qb = dict(self._b[(e, blk)])
        if rows is not None:
            qb = {k: (v[rows] if isinstance(v, np.ndarray) else v) for k, v in qb.items()}
        return qb

    def factors(self, e, blk):
        return self._f.get((e, blk))

    def shared(self, g, blk):
        return self._s.get((g, blk))


def test_toy_closed_form():
    gold = json.load(open(os.path.join(GOLD, "moe_toy_closed_form.json")))
    L = gold["layer"]
    names = {0: "gate", 1: "up", 2: "down"}
    blocks = {}
    for e in range(2):
        for blk in range(3):
            d = L["blocks"][f"e{e}_{names[blk]}"]
            qb = dict(fmt="int", codes=np.array(d["codes"], dtype=np.uint8),
                      s16=np.array(d["s16"], dtype=np.float16), z=np.array(d["z"], dtype=np.uint8))
            assert forward.dequant_int(qb["codes"], qb["s16"], qb["z"], 2).tolist() == d["w_hat"]
            blocks[(e, blk)] = qb
    fac = {(0, 0): (np.array(L["e0_gate_factor"]["U"], dtype=np.float16),
                    np.array(L["e0_gate_factor"]["V"], dtype=np.float16))}
    layer = _DictLayer(2, 2, 2, 2, blocks, fac)
    x = np.array([L["x"]], dtype=np.float16)
    logits = np.array([L["logits"]], dtype=np.float32)
    for case in gold["expected"].values():
        y = forward.moe_forward(layer, x, logits, 2, case["n_comp"])
        assert np.allclose(y[0], case["y"], rtol=0, atol=1e-14)


def _random_layer(rng, E, H, I, G, b, r=0, rs=0, share=0, fmt="int"):
    blocks, fac, sh = {}, {}, {}
    for e in range(E):
        for blk in range(3):
            N, K = (I, H) if blk < 2 else (H, I)
            W = (rng.standard_normal((N, K)) * 0.3).astype(np.float16)
            bb = b if np.isscalar(b) else int(b[e, blk])
            if fmt == "int":
                c, s, z = ptq.rtn_quantize(W, bb, G)
                blocks[(e, blk)] = dict(fmt="int", codes=c, s16=s, z=z)
            else:
                c4, s, z = ptq.rtn_quantize(W, 4, G)
                blocks[(e, blk)] = dict(fmt="bitplane", c4=c4, q=bb,
                                        lut=ptq.bitplane_lut(W, c4, s, z, bb, G))
            if r:
                fac[(e, blk)] = ((rng.standard_normal((N, r)) * 0.1).astype(np.float16),
                                 (rng.standard_normal((r, K)) * 0.1).astype(np.float16))
    if rs:
        for g in range((E + share - 1) // share):
            for blk in range(3):
                N, K = (I, H) if blk < 2 else (H, I)
                sh[(g, blk)] = ((rng.standard_normal((N, rs)) * 0.1).astype(np.float16),
                                (rng.standard_normal((rs, K)) * 0.1).astype(np.float16))
    return _DictLayer(E, H, I, G, blocks, fac, sh, share)


def _brute_dense(layer, x16, logits, k, n_comp):
    """Dense-mask brute force with explicit loops: every expert on every token,
    kept only where the expert is in the token's top-k."""
    T, H = x16.shape
    E, I, G = layer.E, layer.I, layer.G

    def w_hat(qb, n, kk):
        if qb["fmt"] == "int":
            return float(qb["s16"][n, kk // G]) * (int(qb["codes"][n, kk]) - int(qb["z"][n, kk // G]))
        return float(qb["lut"][n, kk // G, int(qb["c4"][n, kk]) >> (4 - qb["q"])])

    def lin(e, blk, v, comp):
        qb = layer.qblock(e, blk)
        N = I if blk < 2 else H
        out = [sum(w_hat(qb, n, kk) * v[kk] for kk in range(len(v))) for n in range(N)]
        if comp:
            for f in (layer.factors(e, blk), layer.shared(layer.group_of(e), blk)):
                if f is None:
                    continue
                U, V = f[0].astype(float), f[1].astype(float)
                zv = [sum(V[i, kk] * v[kk] for kk in range(len(v))) for i in range(V.shape[0])]
                for n in range(N):
                    out[n] += sum(U[n, i] * zv[i] for i in range(len(zv)))
        return out

    y = np.zeros((T, H))
    for t in range(T):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        den = sum(math.exp(row[e] - row[order[0]]) for e in order)
        xt = [float(v) for v in x16[t]]
        for e in range(E):
            if e not in order:
                continue
            j = order.index(e)
            g = math.exp(row[e] - row[order[0]]) / den
            a = lin(e, 0, xt, j < n_comp)
            bb = lin(e, 1, xt, j < n_comp)
            h = [ai / (1 + math.exp(-ai)) * bi for ai, bi in zip(a, bb)]
            yo = lin(e, 2, h, j < n_comp)
            y[t] += g * np.array(yo)
    return y


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("k", [1, 2])
def test_two_expert_toy_brute_force(b, k):
    rng = np.random.default_rng(100 * b + k)
    E, H, I, G, T = 2, 8, 16, 4, 5
    layer = _random_layer(rng, E, H, I, G, b, r=2)
    x = rng.standard_normal((T, H)).astype(np.float16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    for n_comp in (0, 1, k):
        y = forward.moe_forward(layer, x, logits, k, n_comp)
        yb = _brute_dense(layer, x, logits, k, n_comp)
        assert np.allclose(y, yb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", ["int", "bitplane"])
def test_mixed_bits_shared_factors_brute_force(fmt):
    rng = np.random.default_rng(77)
    E, H, I, G, T, k = 4, 8, 8, 4, 6, 3
    bits = rng.choice([2, 3, 4], size=(E, 3))
    layer = _random_layer(rng, E, H, I, G, bits, r=1, rs=2, share=2, fmt=fmt)
    x = rng.standard_normal((T, H)).astype(np.float16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    for n_comp in (0, 2, 3):
        y = forward.moe_forward(layer, x, logits, k, n_comp)
        assert np.allclose(y, _brute_dense(layer, x, logits, k, n_comp), rtol=1e-12, atol=1e-12)


def test_shared_down_term_once_per_token_group():
    """The down side of shared factors applied once per (token, expert
    group) to the gate-weighted sum, sum_e g_e U_G (V_G h_e) =
    U_G (sum_e g_e V_G h_e), gives the routed layer of the per-pair
    definition; the gate/up side's V_G x is the same for every member of a
    (token, group).  Explicit loops over the groups; 8 experts in groups of
    4, top-4, so tokens hit several experts of a group; every n_comp."""
    rng = np.random.default_rng(21)
    E, H, I, G, T, k, share = 8, 16, 24, 8, 10, 4, 4
    layer = _random_layer(rng, E, H, I, G, 3, r=2, rs=3, share=share)
    x = rng.standard_normal((T, H)).astype(np.float16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    rt = forward.route(logits, k)
    for n_comp in (1, 2, 4):
        y = forward.moe_forward(layer, x, logits, k, n_comp)
        y2 = np.zeros((T, H))
        for t in range(T):
            xt = x[t:t + 1].astype(np.float64)
            wsum = {}                 # group -> sum_j g_j V_G h_j over compensated slots
            for j in range(k):
                e, g = int(rt["ids"][t, j]), float(rt["gates"][t, j])
                comp = np.array([j < n_comp])
                grp = layer.group_of(e)
                a = forward.compensated_linear(forward.dequant_block(layer.qblock(e, 0), G), xt, comp,
                                               layer.factors(e, 0), layer.shared(grp, 0))
                b = forward.compensated_linear(forward.dequant_block(layer.qblock(e, 1), G), xt, comp,
                                               layer.factors(e, 1), layer.shared(grp, 1))
                h = forward.silu(a) * b
                # dense and per-expert terms per pair; the shared term deferred
                yp = forward.compensated_linear(forward.dequant_block(layer.qblock(e, 2), G), h, comp,
                                                layer.factors(e, 2), None)
                y2[t] += g * yp[0]
                if j < n_comp:
                    Ug, Vg = (f.astype(np.float64) for f in layer.shared(grp, 2))
                    wsum[grp] = wsum.get(grp, 0.0) + g * (Vg @ h[0])
            for grp, w in wsum.items():
                Ug = layer.shared(grp, 2)[0].astype(np.float64)
                y2[t] += Ug @ w
        assert np.allclose(y2, y, rtol=1e-12, atol=1e-12)
        # some token routes two compensated slots to one group (the case
        # the deduplication changes)
        if n_comp >= 2:
            gi = rt["ids"][:, :n_comp] // share
            assert any(len(set(row)) < n_comp for row in gi.tolist())


def test_compensated_linear_equals_dense_sum():
    """W_hat v + U(V v) + U_G(V_G v) == (W_hat + U V + U_G V_G) v, and rank 0
    (no factors, or comp off) is the plain quantized layer."""
    rng = np.random.default_rng(9)
    W_hat = rng.standard_normal((12, 10))
    v = rng.standard_normal((4, 10))
    U, V = rng.standard_normal((12, 3)).astype(np.float16), rng.standard_normal((3, 10)).astype(np.float16)
    Us, Vs = rng.standard_normal((12, 2)).astype(np.float16), rng.standard_normal((2, 10)).astype(np.float16)
    comp = np.array([True, False, True, True])
    out = forward.compensated_linear(W_hat, v, comp, (U, V), (Us, Vs))
    dense = W_hat + U.astype(float) @ V.astype(float) + Us.astype(float) @ Vs.astype(float)
    assert np.allclose(out[comp], v[comp] @ dense.T, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out[~comp], (v @ W_hat.T)[~comp])
    assert np.array_equal(forward.compensated_linear(W_hat, v, comp, None, None), v @ W_hat.T)
    assert np.array_equal(forward.compensated_linear(W_hat, v, np.zeros(4, bool), (U, V), (Us, Vs)), v @ W_hat.T)
    # shared-only and per-expert-only reduce to the single-factor forms
    a = forward.compensated_linear(W_hat, v, comp, None, (Us, Vs))
    b = forward.compensated_linear(W_hat, v, comp, (Us, Vs), None)
    assert np.array_equal(a, b)


def test_silu_closed_form():
    assert forward.silu(np.array([0.0]))[0] == 0.0
    assert forward.silu(np.array([1.0]))[0] == pytest.approx(math.e / (1 + math.e), rel=1e-15)
    assert forward.silu(np.array([-1.0]))[0] == pytest.approx(-1 / (1 + math.e), rel=1e-15)


def _layer_from_weights(E, H, I, G, b, seed, r=2):
    rng = np.random.default_rng(seed)
    Ws = {(e, blk): (rng.standard_normal((I, H) if blk < 2 else (H, I)) * 0.05).astype(np.float16)
          for e in range(E) for blk in range(3)}
    facs = {(e, blk): ((rng.standard_normal(((I if blk < 2 else H), r)) * 0.05).astype(np.float16),
                       (rng.standard_normal((r, (H if blk < 2 else I))) * 0.05).astype(np.float16))
            for e in range(E) for blk in range(3)}
    return OracleLayer(E, H, I, G, "int", np.full((E, 3), b),
                       lambda e, blk, rows: Ws[(e, blk)] if rows is None else Ws[(e, blk)][rows],
                       factors=lambda e, blk: facs[(e, blk)])


def test_invariants_zero_input_permutation_identical_experts():
    E, H, I, G, T, k = 4, 16, 32, 8, 12, 2
    layer = _layer_from_weights(E, H, I, G, 3, seed=5)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((T, H)).astype(np.float16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # x = 0 -> y = 0
    assert np.all(forward.moe_forward(layer, np.zeros_like(x), logits, k, k) == 0)
    # token permutation: y(P x) = P y(x)
    perm = rng.permutation(T)
    y = forward.moe_forward(layer, x, logits, k, 1)
    yp = forward.moe_forward(layer, x[perm], logits[perm], k, 1)
    assert np.allclose(yp, y[perm], rtol=1e-13, atol=1e-15)
    # identical experts (weights and factors): y = FFN(x) for any routing
    W0 = {blk: (rng.standard_normal((I, H) if blk < 2 else (H, I)) * 0.05).astype(np.float16) for blk in range(3)}
    same = OracleLayer(E, H, I, G, "int", np.full((E, 3), 4),
                       lambda e, blk, rows: W0[blk] if rows is None else W0[blk][rows])
    y = forward.moe_forward(same, x, logits, k, 0)
    y1 = forward.expert_ffn(same, 0, x.astype(np.float64), np.zeros(T, bool))
    assert np.allclose(y, y1, rtol=1e-13, atol=1e-15)


def test_sampled_rows_and_columns_match_full():
    E, H, I, G, T, k = 4, 16, 32, 8, 10, 2
    layer = _layer_from_weights(E, H, I, G, 2, seed=8)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((T, H)).astype(np.float16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    y = forward.moe_forward(layer, x, logits, k, 1)
    toks, cols = np.array([1, 7]), np.array([0, 3, 15])
    ys = forward.moe_forward(layer, x, logits, k, 1, tokens=toks, cols=cols)
    assert np.allclose(ys, y[toks][:, cols], rtol=1e-13, atol=1e-15)


def test_svd_layer_rank0_is_plain_quantized():
    """A layer whose compensators are the truncated SVD of the residual: with
    n_comp = 0 it equals the uncompensated layer exactly, and compensation
    moves every linear closer to the fp16 weights."""
    E, H, I, G, T, k = 2, 32, 64, 16, 6, 2
    rng = np.random.default_rng(12)
    Ws = {(e, blk): (rng.standard_normal((I, H) if blk < 2 else (H, I)) * 0.02).astype(np.float16)
          for e in range(E) for blk in range(3)}
    get = lambda e, blk, rows: Ws[(e, blk)] if rows is None else Ws[(e, blk)][rows]
    svd = OracleLayer(E, H, I, G, "int", np.full((E, 3), 4), get, svd_rank=8)
    plain = OracleLayer(E, H, I, G, "int", np.full((E, 3), 4), get)
    x = rng.standard_normal((T, H)).astype(np.float16)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    assert np.array_equal(forward.moe_forward(svd, x, logits, k, 0),
                          forward.moe_forward(plain, x, logits, k, 0))
    for e in range(E):
        for blk in range(3):
            W = Ws[(e, blk)].astype(np.float64)
            Wh = forward.dequant_block(svd.qblock(e, blk), G)
            U, V = svd.factors(e, blk)
            assert np.linalg.norm(W - Wh - U.astype(float) @ V.astype(float)) < np.linalg.norm(W - Wh)
