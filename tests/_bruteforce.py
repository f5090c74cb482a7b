"""Pure-Python brute force of the MoE layer on tiny inputs (float64 scalars, lists).

Written independently of the oracle to pin it: selection by counting, for every expert,
how many experts beat it (larger logit, or equal logit and lower index); capacity by
walking each expert's tokens in order; the expert FFN and the combine as scalar loops.
Follows the same pages as the oracle (shubhamtatvamasi.com "Mixture of Experts",
sections "The router" and "Load imbalance"; shipai.vats.cc "How routing works").
"""
from __future__ import annotations

import math


def _sig(a):
    return 1.0 / (1.0 + math.exp(-a))


def layer(x, wr, bias, wg, wu, wd, k, gating, cf, shared=()):
    """x [T][d]; wr [E][d]; bias [E] or None; wg/wu [E][f][d]; wd [E][d][f];
    shared: list of (wg [fs][d], wu [fs][d], wd [d][fs]). Lists of floats."""
    T, d, E = len(x), len(x[0]), len(wr)
    logits = [[sum(float(x[t][i]) * float(wr[e][i]) for i in range(d)) + (float(bias[e]) if bias is not None else 0.0)
               for e in range(E)] for t in range(T)]
    idx, gate = [], []
    for t in range(T):
        l = logits[t]
        ranked = []
        for e in range(E):
            beaten_by = sum(1 for i in range(E) if l[i] > l[e] or (l[i] == l[e] and i < e))
            if beaten_by < k:
                ranked.append((beaten_by, e))
        ranked.sort()
        chosen = [e for _, e in ranked]
        if gating == "softmax":
            w = [math.exp(l[e]) for e in chosen]
        else:
            w = [_sig(l[e]) for e in chosen]
        s = sum(w)
        idx.append(chosen)
        gate.append([v / s for v in w])
    cap = None
    if cf > 0:
        cap = math.ceil(float(cf) * float(T * k) / float(E))
    kept = [[True] * k for _ in range(T)]
    for e in range(E):
        seen = 0
        for t in range(T):
            for j in range(k):
                if idx[t][j] == e:
                    seen += 1
                    if cap is not None and seen > cap:
                        kept[t][j] = False

    def ffn(v, g, u, dn):
        f = len(g)
        h = []
        for n in range(f):
            a = sum(v[i] * float(g[n][i]) for i in range(d))
            b = sum(v[i] * float(u[n][i]) for i in range(d))
            h.append(a * _sig(a) * b)
        return [sum(h[n] * float(dn[o][n]) for n in range(f)) for o in range(d)]

    y = []
    for t in range(T):
        v = [float(a) for a in x[t]]
        acc = [0.0] * d
        for j in range(k):
            if kept[t][j]:
                e = idx[t][j]
                o = ffn(v, wg[e], wu[e], wd[e])
                for i in range(d):
                    acc[i] += gate[t][j] * o[i]
        for (g, u, dn) in shared:
            o = ffn(v, g, u, dn)
            for i in range(d):
                acc[i] += o[i]
        y.append(acc)
    return dict(logits=logits, idx=idx, gate=gate, kept=kept, capacity=cap, y=y)
