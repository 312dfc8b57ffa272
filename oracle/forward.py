"""Oracle forward pass of the routed low-bit MoE expert layer (test
infrastructure only; see ``oracle/__init__.py``).

What is computed, with the passage each step follows:

* Routing.  Each token keeps its k largest router logits (MoE top-k routing
  named in the PagedWeight review, "Where Pith is reading between the lines" /
  "If this is right": MoE architectures with different expert counts and
  top-k choices).  Readings: ties go to the lower expert id; the k experts are
  ordered by descending logit; the gates are the softmax over the k selected
  logits (equal to the renormalised full softmax, so they sum to 1).
* Router-guided compensation (Bandwidth-Efficient Adaptive MoE abstract:
  compensation only for the top-n, n < k, experts of each token).  Reading:
  the first n_comp slots of a token's top-k list are compensated, for all
  three linears of that expert.
* Counting sort of (token, slot) pairs by expert, stable in the flat pair id
  p = t * k + j, with prefix-sum offsets (MxMoE abstract: heterogeneous work
  per expert from divergent activation frequency).
* Dequantization: INT  w_hat = s16 * (c - z);  bit-plane  w_hat = LUT[i] with
  i = c4 >> (4 - q) (PagedWeight Figure 3 caption).
* Compensated linear (MiLo abstract; TileQ abstract for factors shared across
  a group of experts):  L(v) = W_hat v + [comp] (U (V v) + U_G (V_G v)).
* SwiGLU expert FFN and gate-weighted combine:
      h = SiLU(L_gate x) * L_up x,  SiLU(a) = a / (1 + exp(-a)),
      y_t = sum_j g_{t,j} L_down(h_{t,j})   (summed in slot order j = 0..k-1).

All arithmetic is float64 on the stored fp16 / uint8 parameters.
"""

import numpy as np

GATE, UP, DOWN = 0, 1, 2


# ----------------------------------------------------------------- routing

def topk_ids(logits, k):
    """Per token, the k expert ids with the largest logits, ordered by
    descending logit, ties broken toward the lower expert id."""
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    eid = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((eid, -l), axis=1)    # primary key -logit, then id
    return order[:, :k].astype(np.int32)


def gates_of(logits, ids):
    """Softmax over the selected logits of each token (float64)."""
    l = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    e = np.exp(sel - sel[:, :1])
    return e / e.sum(axis=1, keepdims=True)


def counting_sort(ids_flat, E):
    """Stable counting sort of pair ids by expert.

    Returns (offsets [E+1], sorted_pairs [P], pair_pos [P]), all int32:
    offsets is the exclusive prefix sum of the per-expert counts, the pairs of
    expert e occupy sorted_pairs[offsets[e]:offsets[e+1]] in ascending pair
    id, and pair_pos is the inverse permutation.
    """
    ids_flat = np.asarray(ids_flat, dtype=np.int64)
    P = ids_flat.shape[0]
    counts = np.zeros(E, dtype=np.int64)
    for e in ids_flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_pairs = np.empty(P, dtype=np.int64)
    pair_pos = np.empty(P, dtype=np.int64)
    for p in range(P):
        e = ids_flat[p]
        sorted_pairs[cursor[e]] = p
        pair_pos[p] = cursor[e]
        cursor[e] += 1
    return offsets.astype(np.int32), sorted_pairs.astype(np.int32), pair_pos.astype(np.int32)


def route(logits, k):
    """Top-k routing, gates and the expert counting sort of one layer call."""
    logits = np.asarray(logits)
    T, E = logits.shape
    ids = topk_ids(logits, k)
    gates = gates_of(logits, ids)
    offsets, sorted_pairs, pair_pos = counting_sort(ids.reshape(-1), E)
    return dict(ids=ids, gates=gates, offsets=offsets,
                sorted_pairs=sorted_pairs, pair_pos=pair_pos)


def routing_mass(ids, gates, E):
    """Gate-weighted routing mass of each expert: m_e = sum over (t, j) with
    ids[t, j] == e of gates[t, j] (float64), the per-expert usage measure
    that PagedWeight's planner buckets ("Routing-mass buckets", review
    summary; the planner's routing-bucket multiplier)."""
    m = np.zeros(E, dtype=np.float64)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            m[int(ids[t, j])] += float(gates[t, j])
    return m


def mass_bucket(mass, edges):
    """Bucket index of each mass against ascending edges: the number of
    edges that are <= the mass (bucket b holds edges[b-1] <= m < edges[b])."""
    edges = np.asarray(edges, dtype=np.float64)
    return np.array([int(np.sum(edges <= m)) for m in np.asarray(mass)], dtype=np.int32)


# ----------------------------------------------------------------- dequant

def dequant_int(codes, s16, z, G):
    """w_hat[n, k] = s16[n, k // G] * (codes[n, k] - z[n, k // G]) in float64."""
    codes = np.asarray(codes, dtype=np.float64)
    N, K = codes.shape
    s = np.repeat(np.asarray(s16, dtype=np.float64), G, axis=1)
    zz = np.repeat(np.asarray(z, dtype=np.float64), G, axis=1)
    assert s.shape == (N, K)
    return s * (codes - zz)


def dequant_bitplane(c4, lut, q, G):
    """w_hat[n, k] = lut[n, k // G, c4[n, k] >> (4 - q)] in float64."""
    c4 = np.asarray(c4, dtype=np.int64)
    N, K = c4.shape
    idx = c4 >> (4 - q)
    grp = np.broadcast_to(np.arange(K) // G, (N, K))
    rows = np.broadcast_to(np.arange(N)[:, None], (N, K))
    return np.asarray(lut, dtype=np.float64)[rows, grp, idx]


def dequant_block(qb, G):
    """Dense float64 W_hat of a quantized block description (see layer.py)."""
    if qb["fmt"] == "int":
        return dequant_int(qb["codes"], qb["s16"], qb["z"], G)
    return dequant_bitplane(qb["c4"], qb["lut"], qb["q"], G)


# ----------------------------------------------------------------- FFN

def silu(a):
    return a / (1.0 + np.exp(-a))


def compensated_linear(W_hat, v, comp, fac=None, shared=None):
    """L(v) = W_hat v + comp * (U (V v) + U_G (V_G v)) for the rows v [m, K].

    comp is a boolean mask over the m rows; fac / shared are (U, V) pairs of
    fp16 factors or None.
    """
    out = v @ W_hat.T
    comp = np.asarray(comp, dtype=bool)
    for f in (fac, shared):
        if f is None or not comp.any():
            continue
        U = np.asarray(f[0], dtype=np.float64)
        V = np.asarray(f[1], dtype=np.float64)
        if U.shape[1] == 0:
            continue
        low = (v[comp] @ V.T) @ U.T
        out[comp] += low
    return out


def expert_ffn(layer, e, xs, comp, down_rows=None):
    """Expert e on token rows xs [m, H] float64: Down(SiLU(Gate x) * Up x).

    down_rows restricts the output to selected rows of the down block
    (output channels), for sampled checks of large layers.
    """
    G = layer.G
    grp = layer.group_of(e)
    a = compensated_linear(dequant_block(layer.qblock(e, GATE), G), xs, comp,
                           layer.factors(e, GATE), layer.shared(grp, GATE))
    b = compensated_linear(dequant_block(layer.qblock(e, UP), G), xs, comp,
                           layer.factors(e, UP), layer.shared(grp, UP))
    h = silu(a) * b
    fac = layer.factors(e, DOWN)
    sh = layer.shared(grp, DOWN)
    if down_rows is not None:
        down_rows = np.asarray(down_rows)
        if fac is not None:
            fac = (fac[0][down_rows], fac[1])
        if sh is not None:
            sh = (sh[0][down_rows], sh[1])
    Wd = dequant_block(layer.qblock(e, DOWN, rows=down_rows), G)
    return compensated_linear(Wd, h, comp, fac, sh)


def moe_forward(layer, x16, logits, k, n_comp, tokens=None, cols=None, routing=None):
    """y [T, H] float64 of the routed layer (or y[tokens][:, cols]).

    x16: fp16 activations [T, H]; logits: fp32 [T, E]; n_comp: number of
    leading top-k slots that get the low-rank compensation.
    """
    x = np.asarray(x16, dtype=np.float64)
    T = x.shape[0]
    rt = routing if routing is not None else route(logits, k)
    ids, gates = rt["ids"], rt["gates"]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    ncols = layer.H if cols is None else len(cols)
    # y_pair for every (token, slot) pair of the selected tokens, per expert
    ypair = {}
    for e in range(layer.E):
        sel = [(int(t), j) for t in tokens for j in range(k) if ids[t, j] == e]
        if not sel:
            continue
        xs = x[[t for t, _ in sel]]
        comp = np.array([j < n_comp for _, j in sel])
        ye = expert_ffn(layer, e, xs, comp, down_rows=cols)
        for (t, j), row in zip(sel, ye):
            ypair[(t, j)] = row
    y = np.zeros((len(tokens), ncols), dtype=np.float64)
    for i, t in enumerate(tokens):
        for j in range(k):
            y[i] += gates[t, j] * ypair[(int(t), j)]
    return y
