"""Pins of the oracle's backward pass (oracle.backward) against things other than itself:

* torch autograd, in float64 on the CPU, through a forward written here with torch's own
  operations (its own softmax, sigmoid, silu and matrix products, its own capacity walk);
* central finite differences of the scalar loss sum(y * dy) + L_aux, the definition of the
  derivative, on inputs whose top-k choices are far from ties;
* closed forms: under softmax gating the logit gradient of every token sums to zero; the
  load-balancing loss is aux_coef when the router is uniform, with a zero gradient.

Pages: techbonafide.com "Mixture of Experts (MoE) Explained" ("Challenges and Tradeoffs":
auxiliary losses, after the Switch Transformer work); shipai.vats.cc "Mixture of Experts
(MoE)" (training adds load-balancing losses); shubhamtatvamasi.com/llm-inference/moe
("The router", "Load imbalance").
"""
import math

import numpy as np
import pytest
import torch

import oracle


def make_case(seed, T=13, d=16, f=24, E=5, k=2, n_shared=0, fs=16, bias=True, spread=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) * spread / math.sqrt(d)
    b = rng.standard_normal(E) * 0.3 if bias else None
    ex = [(rng.standard_normal((f, d)) / math.sqrt(d), rng.standard_normal((f, d)) / math.sqrt(d),
           rng.standard_normal((d, f)) / math.sqrt(f)) for _ in range(E)]
    sh = [(rng.standard_normal((fs, d)) / math.sqrt(d), rng.standard_normal((fs, d)) / math.sqrt(d),
           rng.standard_normal((d, fs)) / math.sqrt(fs)) for _ in range(n_shared)]
    dy = rng.standard_normal((T, d))
    return x, wr, b, ex, sh, dy


def torch_loss(x, wr, b, ex, sh, dy, idx, k, gating, cf, aux_coef):
    """sum(y * dy) + L_aux with torch operations; the routing decision idx is given."""
    T, E = x.shape[0], wr.shape[0]
    logits = x @ wr.T + (b if b is not None else 0.0)
    sel = torch.gather(logits, 1, idx)
    if gating == "softmax":
        g = torch.softmax(sel, dim=1)
    else:
        s = torch.sigmoid(sel)
        g = s / s.sum(dim=1, keepdim=True)
    # capacity: walk each expert's pairs in token order, keep the first C
    keep = torch.ones_like(idx, dtype=torch.bool)
    if cf > 0:
        C = math.ceil(float(np.float32(cf)) * T * k / E)
        for e in range(E):
            n = 0
            for t in range(T):
                for j in range(k):
                    if int(idx[t, j]) == e:
                        n += 1
                        if n > C:
                            keep[t, j] = False
    y = torch.zeros_like(x)
    for e in range(E):
        wg, wu, wd = ex[e]
        for j in range(k):
            m = (idx[:, j] == e) & keep[:, j]
            if m.any():
                v = x[m]
                h = torch.nn.functional.silu(v @ wg.T) * (v @ wu.T)
                y = y.index_add(0, torch.nonzero(m).flatten(), g[m, j, None] * (h @ wd.T))
    for wg, wu, wd in sh:
        y = y + (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T
    loss = (y * dy).sum()
    if aux_coef:
        counts = torch.bincount(idx.flatten(), minlength=E).to(x.dtype)
        f = counts / (T * k)
        p = torch.softmax(logits, dim=1) if gating == "softmax" else \
            torch.sigmoid(logits) / torch.sigmoid(logits).sum(dim=1, keepdim=True)
        loss = loss + aux_coef * E * (f * p.mean(dim=0)).sum()
    return loss


CASES = [
    dict(gating="softmax", cf=0.0, aux=0.0, n_shared=0),
    dict(gating="sigmoid", cf=0.0, aux=0.0, n_shared=1),
    dict(gating="softmax", cf=0.7, aux=0.01, n_shared=0),
    dict(gating="sigmoid", cf=0.5, aux=0.05, n_shared=2),
    dict(gating="softmax", cf=0.0, aux=0.1, n_shared=1, k=5),  # k = E: the dense mixture
    dict(gating="sigmoid", cf=0.0, aux=0.0, n_shared=0, k=1),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=lambda i: "_".join(f"{k}{v}" for k, v in CASES[i].items()))
def test_backward_matches_torch_autograd(ci):
    c = CASES[ci]
    k = c.get("k", 2)
    x, wr, b, ex, sh, dy = make_case(100 + ci, n_shared=c["n_shared"], k=k)
    ref = oracle.backward(x, wr, b, dy, top_k=k, gating=c["gating"], capacity_factor=c["cf"], experts=ex,
                          shared=sh, n_shared=c["n_shared"], aux_coef=c["aux"])
    if c["cf"] > 0:
        assert ref["pos"].min() < 0, "the capacity case should drop some pairs"
    tt = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
    X, WR, B = tt(x), tt(wr), tt(b)
    EX = [tuple(tt(w) for w in e) for e in ex]
    SH = [tuple(tt(w) for w in s) for s in sh]
    loss = torch_loss(X, WR, B, EX, SH, torch.tensor(dy), torch.tensor(ref["idx"]), k, c["gating"], c["cf"],
                      c["aux"])
    params = [X, WR, B] + [w for e in EX for w in e] + [w for s in SH for w in s]
    grads = torch.autograd.grad(loss, params, allow_unused=True)
    got = [ref["dx"], ref["dw_router"], ref["db_router"]]
    for e in range(len(ex)):
        got += [ref["dw_gate"][e], ref["dw_up"][e], ref["dw_down"][e]]
    for s in range(len(sh)):
        got += [ref["dws_gate"][s], ref["dws_up"][s], ref["dws_down"][s]]
    for i, (g_t, g_o) in enumerate(zip(grads, got)):
        g_t = np.zeros_like(g_o) if g_t is None else g_t.numpy()
        np.testing.assert_allclose(g_o, g_t, rtol=1e-10, atol=1e-12, err_msg=f"parameter {i}")
    if c["aux"]:
        T, E = x.shape[0], wr.shape[0]
        counts = np.bincount(ref["idx"].ravel(), minlength=E)
        _, aux_only = oracle.aux_loss(ref["logits"], counts, k, c["gating"], c["aux"])
        assert np.abs(aux_only).max() > 0


def _loss_np(x, wr, b, ex, sh, dy, k, gating, cf, aux):
    out = oracle.forward(x, wr, b, top_k=k, gating=gating, capacity_factor=cf, experts=ex, shared=sh,
                         n_shared=len(sh))
    loss = float((out["y"] * dy).sum())
    if aux:
        loss += oracle.aux_loss(out["logits"], out["counts"], k, gating, aux)[0]
    return loss, out["idx"]


@pytest.mark.parametrize("gating,cf,aux,n_shared", [("softmax", 0.0, 0.02, 1), ("sigmoid", 0.6, 0.05, 1)])
def test_backward_matches_central_differences(gating, cf, aux, n_shared):
    k = 2
    x, wr, b, ex, sh, dy = make_case(11, T=9, d=8, f=12, E=4, n_shared=n_shared, fs=8, spread=4.0)
    ref = oracle.backward(x, wr, b, dy, top_k=k, gating=gating, capacity_factor=cf, experts=ex, shared=sh,
                          n_shared=n_shared, aux_coef=aux)
    # the choice must stay put under the perturbation: every k-th/(k+1)-th gap is wide
    srt = -np.sort(-ref["logits"], axis=1)
    assert (srt[:, k - 1] - srt[:, k]).min() > 1e-3
    rng = np.random.default_rng(3)
    eps = 1e-6
    targets = [("x", x, ref["dx"]), ("wr", wr, ref["dw_router"]), ("b", b, ref["db_router"])]
    for e in range(4):
        targets += [(f"wg{e}", ex[e][0], ref["dw_gate"][e]), (f"wd{e}", ex[e][2], ref["dw_down"][e])]
    targets += [("swu0", sh[0][1], ref["dws_up"][0])]
    for name, arr, grad in targets:
        for _ in range(3):
            i = tuple(int(rng.integers(0, n)) for n in arr.shape)
            old = arr[i]
            arr[i] = old + eps
            lp, idx_p = _loss_np(x, wr, b, ex, sh, dy, k, gating, cf, aux)
            arr[i] = old - eps
            lm, idx_m = _loss_np(x, wr, b, ex, sh, dy, k, gating, cf, aux)
            arr[i] = old
            assert (idx_p == ref["idx"]).all() and (idx_m == ref["idx"]).all()
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, grad[i])


def test_softmax_logit_gradient_sums_to_zero_per_token():
    x, wr, b, ex, sh, dy = make_case(5, n_shared=1)
    r = oracle.backward(x, wr, b, dy, top_k=2, gating="softmax", capacity_factor=0.8, experts=ex, shared=sh,
                        n_shared=1, aux_coef=0.1)
    np.testing.assert_allclose(r["dl"].sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(r["db_router"].sum(), 0.0, atol=1e-11)


def test_aux_loss_of_a_uniform_router_is_the_coefficient_with_zero_gradient():
    T, E, k = 12, 6, 3
    logits = np.zeros((T, E))
    counts = np.full(E, T * k // E)  # every expert gets T k / E pairs
    for gating in ("softmax", "sigmoid"):
        loss, dl = oracle.aux_loss(logits, counts, k, gating, 0.25)
        assert abs(loss - 0.25) < 1e-15
        np.testing.assert_allclose(dl, 0.0, atol=1e-18)


def test_aux_loss_of_a_collapsed_router():
    """Every pair on expert 0 (f = [1/k ... ]) with a router certain of expert 0 (p -> 1):
    L_aux -> aux_coef * E * f_0 = aux_coef * E / k when each token sends one of its k pairs there."""
    T, E, k = 10, 8, 2
    logits = np.full((T, E), -60.0)
    logits[:, 0] = 60.0
    counts = np.zeros(E, int)
    counts[0] = T
    counts[1] = T
    loss, _ = oracle.aux_loss(logits, counts, k, "softmax", 1.0)
    assert abs(loss - E * 0.5) < 1e-9


def test_single_expert_router_gets_no_gate_gradient():
    """E = k = 1: the gate is identically 1, so no gradient reaches the router."""
    x, wr, b, ex, sh, dy = make_case(9, E=1, k=1)
    r = oracle.backward(x, wr, b, dy, top_k=1, gating="softmax", capacity_factor=0.0, experts=ex)
    assert np.abs(r["dw_router"]).max() == 0 and np.abs(r["db_router"]).max() == 0
