"""Oracle of the bitwidth-reduction planner (test infrastructure only; see
``oracle/__init__.py``).

PagedWeight review page ("What carries the argument"; referee summary): a
weight page is one bit-plane of an expert linear block with its lookup
table; under memory pressure the planner turns a byte target into page
releases, choosing by predicted damage per released byte, with the damage
of an action d = max(eps, mu_beta * g_i * eta_i) (sensitivity g_i, routing-
bucket multiplier mu_beta, prompt-residual factor eta_i, floor eps).

Reading (the pages give no table layout): an action lowers one block's
committed bit-plane count q by one (releasing one plane and shrinking its
table); g is given per block and resulting bitwidth, g[i][q - 2] for q in
2..4; bytes[i][q - 2] are the block's page bytes at q.  The greedy takes,
while the released bytes are below the target, the available action with
the smallest damage / released bytes (ties: lower block index); a target
<= 0 takes no action; the floor is q = 2.
"""

import itertools

import numpy as np


def action(i, q, bytes_tbl, g, mu, eta, eps):
    """(damage, released bytes) of lowering block i from q to q - 1."""
    rel = float(bytes_tbl[i][q - 2] - bytes_tbl[i][q - 3])
    dmg = max(eps, float(mu[i]) * float(g[i][q - 3]) * float(eta[i]))
    return dmg, rel


def greedy_plan(q, bytes_tbl, g, mu, eta, eps, target):
    q = [int(v) for v in q]
    order, released, damage = [], 0.0, 0.0
    if target <= 0:
        return q, order, released, damage
    while released < target:
        best = None
        for i in range(len(q)):
            if q[i] <= 2:
                continue
            d, r = action(i, q[i], bytes_tbl, g, mu, eta, eps)
            key = d / r
            if best is None or key < best[0]:
                best = (key, i, d, r)
        if best is None:
            break
        _, i, d, r = best
        q[i] -= 1
        order.append(i)
        released += r
        damage += d
    return q, order, released, damage


def exact_plan(q, bytes_tbl, g, mu, eta, eps, target):
    """Least total damage over every assignment of final bitwidths (each
    block lowered step by step from its q) that releases >= target bytes;
    brute force, tiny inputs only.  Returns (damage, released) or None."""
    best = None
    choices = [range(2, int(v) + 1) for v in q]
    for final in itertools.product(*choices):
        dmg, rel = 0.0, 0.0
        for i, (q0, q1) in enumerate(zip(q, final)):
            for qq in range(int(q0), q1, -1):
                d, r = action(i, qq, bytes_tbl, g, mu, eta, eps)
                dmg += d
                rel += r
        if rel >= target and (best is None or dmg < best[0]):
            best = (dmg, rel)
    return best
