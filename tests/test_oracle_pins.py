"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test ties the oracle to something other than itself: a pure-Python brute force,
a library routine the special case reduces to (scipy's softmax/expit, torch's linear and
silu on the CPU), an exact invariant, or the closed form the pages print for the
fraction of experts touched ("Memory vs compute, quantified",
shubhamtatvamasi.com/llm-inference/moe).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from tests import _bruteforce as bf


def _rng(*s):
    return np.random.default_rng(list(s))


def _dense_ffn_torch(x, wg, wu, wd):
    """Textbook SwiGLU block through torch's CPU linear/silu in float64."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    xv = t(x)
    return F.linear(F.silu(F.linear(xv, t(wg))) * F.linear(xv, t(wu)), t(wd)).numpy()


# ------------------------------------------------------------------ brute force
def _tiny_case(seed, T, E, d, f, integer):
    r = _rng(7, seed)
    if integer:  # small integers: integer logits, so exact ties are common
        x = r.integers(-2, 3, (T, d)).astype(np.float64)
        wr = r.integers(-1, 2, (E, d)).astype(np.float64)
    else:
        x = r.standard_normal((T, d))
        wr = r.standard_normal((E, d))
    wg = r.standard_normal((E, f, d)) * 0.5
    wu = r.standard_normal((E, f, d)) * 0.5
    wd = r.standard_normal((E, d, f)) * 0.5
    return x, wr, wg, wu, wd


CASES = []
for seed, (T, E, d, f) in enumerate([(4, 4, 4, 3), (3, 3, 2, 2), (4, 2, 3, 3), (1, 4, 4, 1), (4, 1, 2, 2)]):
    for k in range(1, E + 1):
        for gating in ("softmax", "sigmoid"):
            for cf in (0.0, 0.5, 1.0):
                for integer in (True, False):
                    CASES.append((seed, T, E, d, f, k, gating, cf, integer))


@pytest.mark.parametrize("seed,T,E,d,f,k,gating,cf,integer", CASES)
def test_oracle_matches_bruteforce(seed, T, E, d, f, k, gating, cf, integer):
    x, wr, wg, wu, wd = _tiny_case(seed, T, E, d, f, integer)
    bias = None if seed % 2 else _rng(8, seed).standard_normal(E)
    sh = []
    if seed == 0:
        r = _rng(9, seed)
        sh = [(r.standard_normal((2, d)), r.standard_normal((2, d)), r.standard_normal((d, 2)))]
    want = bf.layer(x.tolist(), wr.tolist(), None if bias is None else bias.tolist(),
                    wg.tolist(), wu.tolist(), wd.tolist(), k, gating, cf,
                    [tuple(m.tolist() for m in s) for s in sh])
    got = oracle.forward(x, wr, bias, top_k=k, gating=gating, capacity_factor=cf,
                         experts=list(zip(wg, wu, wd)), shared=sh, n_shared=len(sh))
    assert got["idx"].tolist() == want["idx"]
    np.testing.assert_allclose(got["gate"], np.array(want["gate"]), rtol=1e-12, atol=1e-14)
    assert got["capacity"] == want["capacity"]
    np.testing.assert_array_equal(got["drop"].reshape(T, k) == 0, np.array(want["kept"]))
    np.testing.assert_allclose(got["y"], np.array(want["y"]), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------ selection
def test_zero_router_ties_go_to_lowest_index():
    x = _rng(1).standard_normal((16, 8))
    for E in (4, 8, 32):
        for k in range(1, E + 1, 3):
            idx, gate, _ = oracle.route(x, np.zeros((E, 8)), None, k, "softmax")
            assert (idx == np.arange(k)[None, :]).all()
            np.testing.assert_allclose(gate, 1.0 / k, rtol=0, atol=1e-15)


def test_exactly_k_distinct_descending():
    l = _rng(2).integers(-3, 4, (500, 16)).astype(np.float64)  # many ties
    for k in (1, 2, 5, 16):
        idx = oracle.select_topk(l, k)
        for t in range(len(l)):
            assert len(set(idx[t])) == k
            sel = l[t, idx[t]]
            # descending logits, ties in ascending expert order
            for a, b in zip(range(k - 1), range(1, k)):
                assert sel[a] > sel[b] or (sel[a] == sel[b] and idx[t, a] < idx[t, b])
            # nothing left out beats the k-th choice
            rest = np.setdiff1d(np.arange(16), idx[t])
            kth_l, kth_e = sel[-1], idx[t, -1]
            assert not any(l[t, e] > kth_l or (l[t, e] == kth_l and e < kth_e) for e in rest)


# ------------------------------------------------------------------ gates
@pytest.mark.parametrize("gating", ["softmax", "sigmoid"])
def test_gates_sum_to_one(gating):
    l = _rng(3).standard_normal((1000, 64)) * 4
    for k in (1, 2, 8, 64):
        idx = oracle.select_topk(l, k)
        g = oracle.gate_values(l, idx, gating)
        assert np.abs(g.sum(1) - 1).max() <= 1e-12
        assert (g > 0).all()
        if k == 1:
            assert (g == 1.0).all()


def test_softmax_renorm_equals_full_softmax_renormalised():
    l = _rng(4).standard_normal((200, 32)) * 3
    for k in (1, 2, 8, 32):
        idx = oracle.select_topk(l, k)
        p = np.take_along_axis(scipy.special.softmax(l, axis=1), idx, 1)
        np.testing.assert_allclose(oracle.gate_values(l, idx, "softmax"), p / p.sum(1, keepdims=True),
                                   rtol=1e-13)
        if k == 32:
            np.testing.assert_allclose(np.take_along_axis(oracle.gate_values(l, idx, "softmax"),
                                                          np.argsort(idx, 1), 1),
                                       scipy.special.softmax(l, axis=1), rtol=1e-13)


def test_sigmoid_renorm_matches_expit():
    l = _rng(5).standard_normal((200, 32)) * 3
    for k in (1, 4, 8, 32):
        idx = oracle.select_topk(l, k)
        s = scipy.special.expit(np.take_along_axis(l, idx, 1))
        np.testing.assert_allclose(oracle.gate_values(l, idx, "sigmoid"), s / s.sum(1, keepdims=True),
                                   rtol=1e-13)


# ------------------------------------------------------------------ layer special cases
def _experts(seed, E, d, f):
    r = _rng(10, seed)
    return [(r.standard_normal((f, d)) / math.sqrt(d), r.standard_normal((f, d)) / math.sqrt(d),
             r.standard_normal((d, f)) / math.sqrt(f)) for _ in range(E)]


def test_k_equals_E_softmax_is_dense_mixture():
    """k = E with softmax: y = sum_e softmax(l)_e FFN_e(x), the dense mixture."""
    T, d, f, E = 24, 16, 12, 6
    x = _rng(11).standard_normal((T, d))
    wr = _rng(12).standard_normal((E, d))
    b = _rng(13).standard_normal(E)
    ex = _experts(1, E, d, f)
    got = oracle.forward(x, wr, b, top_k=E, gating="softmax", capacity_factor=0, experts=ex)["y"]
    p = scipy.special.softmax(x @ wr.T + b, axis=1)
    want = sum(p[:, e:e + 1] * _dense_ffn_torch(x, *ex[e]) for e in range(E))
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("gating", ["softmax", "sigmoid"])
def test_one_hot_router_is_single_dense_ffn(gating):
    T, d, f, E = 20, 16, 12, 5
    x = _rng(14).standard_normal((T, d))
    ex = _experts(2, E, d, f)
    for hot in range(E):
        b = np.full(E, -50.0)
        b[hot] = 50.0
        got = oracle.forward(x, np.zeros((E, d)), b, top_k=1, gating=gating, capacity_factor=0,
                             experts=ex)
        assert (got["idx"][:, 0] == hot).all()
        np.testing.assert_allclose(got["y"], _dense_ffn_torch(x, *ex[hot]), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("gating,k", [("softmax", 2), ("softmax", 4), ("sigmoid", 3)])
def test_identical_experts_give_the_dense_ffn(gating, k):
    """Gates sum to one, so identical experts make routing irrelevant (dropless)."""
    T, d, f, E = 40, 16, 24, 8
    x = _rng(15).standard_normal((T, d))
    w = _experts(3, 1, d, f)[0]
    got = oracle.forward(x, _rng(16).standard_normal((E, d)), None, top_k=k, gating=gating,
                         capacity_factor=0, experts=[w] * E)
    np.testing.assert_allclose(got["y"], _dense_ffn_torch(x, *w), rtol=1e-11, atol=1e-12)


def test_shared_expert_added_with_weight_one():
    T, d, f, E = 10, 8, 6, 4
    x = _rng(17).standard_normal((T, d))
    ex = _experts(4, E, d, f)
    sh = _experts(5, 2, d, f)
    base = oracle.forward(x, _rng(18).standard_normal((E, d)), None, top_k=2, gating="sigmoid",
                          capacity_factor=0, experts=ex)
    withs = oracle.forward(x, _rng(18).standard_normal((E, d)), None, top_k=2, gating="sigmoid",
                           capacity_factor=0, experts=ex, shared=sh, n_shared=2)
    np.testing.assert_allclose(withs["y"] - base["y"],
                               _dense_ffn_torch(x, *sh[0]) + _dense_ffn_torch(x, *sh[1]),
                               rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------ capacity and permutation
def _skewed_idx(seed, T, E, k):
    l = _rng(19, seed).standard_normal((T, E)) + np.linspace(3, -3, E)[None, :]
    return oracle.select_topk(l, k)


@pytest.mark.parametrize("T,E,k,cf", [(512, 16, 2, 1.25), (300, 8, 3, 0.7), (1000, 32, 8, 1.0),
                                      (64, 4, 4, 2.0)])
def test_capacity_keeps_lowest_tokens_within_bound(T, E, k, cf):
    idx = _skewed_idx(T, T, E, k)
    C = oracle.expert_capacity(cf, T, k, E)
    assert C == math.ceil(cf * T * k / E)
    p = oracle.permute(idx, E, C)
    kept = p["drop"].reshape(T, k) == 0
    for e in range(E):
        toks = [t for t in range(T) for j in range(k) if idx[t, j] == e]
        kept_toks = [t for t in range(T) for j in range(k) if idx[t, j] == e and kept[t, j]]
        assert toks == sorted(toks)
        assert kept_toks == toks[:C]  # the lowest token indices survive
        assert len(kept_toks) <= C
        assert p["counts"][e] == len(toks)
        assert p["offsets"][e + 1] - p["offsets"][e] == min(len(toks), C)


def test_large_capacity_factor_is_dropless():
    T, E, k = 400, 16, 4
    idx = _skewed_idx(1, T, E, k)
    C = oracle.expert_capacity(E / k, T, k, E)
    assert C >= T
    a, b = oracle.permute(idx, E, C), oracle.permute(idx, E, None)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_capacity_none_when_factor_not_positive():
    for cf in (0.0, -1.0):
        assert oracle.expert_capacity(cf, 100, 2, 8) is None


def test_tiny_capacity_leaves_shared_only_for_dropped_tokens():
    T, d, f, E, k = 12, 8, 6, 2, 1
    x = _rng(20).standard_normal((T, d))
    ex, sh = _experts(6, E, d, f), _experts(7, 1, d, f)
    out = oracle.forward(x, _rng(21).standard_normal((E, d)), None, top_k=k, gating="softmax",
                         capacity_factor=0.01, experts=ex, shared=sh, n_shared=1)
    assert out["capacity"] == 1
    dropped = out["drop"].reshape(T, k)[:, 0] == 1
    assert dropped.sum() == T - len(np.unique(out["idx"]))  # one kept token per used expert
    np.testing.assert_allclose(out["y"][dropped], _dense_ffn_torch(x[dropped], *sh[0]), rtol=1e-12)


@pytest.mark.parametrize("T,E,k,cf", [(777, 8, 2, 0), (777, 8, 2, 1.1), (2048, 64, 8, 0), (2048, 64, 8, 1.25)])
def test_permutation_invariants(T, E, k, cf):
    idx = _skewed_idx(2, T, E, k)
    C = oracle.expert_capacity(cf, T, k, E)
    p = oracle.permute(idx, E, C)
    n_kept = int(p["offsets"][-1])
    assert p["counts"].sum() == T * k
    assert (np.diff(p["offsets"]) >= 0).all() and p["offsets"][0] == 0
    if C is None:
        assert n_kept == T * k and not p["drop"].any()
    kept = np.flatnonzero(p["pos"] >= 0)
    assert len(kept) == n_kept
    assert sorted(p["pos"][kept].tolist()) == list(range(n_kept))  # bijection
    np.testing.assert_array_equal(p["sorted_slot"][p["pos"][kept]], kept)
    flat = idx.reshape(-1)
    for e in range(E):
        seg = p["sorted_slot"][p["offsets"][e]:p["offsets"][e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg // k) > 0).all()  # ascending token within the expert


# ------------------------------------------------------------------ experts touched
@pytest.mark.parametrize("E,k,T", [(8, 2, 1), (8, 2, 4), (8, 2, 16), (8, 2, 64), (128, 8, 1),
                                   (128, 8, 4), (128, 8, 16)])
def test_experts_touched_matches_closed_form(E, k, T):
    """Uniform routing (iid logits): expected touched fraction is 1 - (1 - k/E)^T."""
    trials = 2000
    l = _rng(22, E, k, T).standard_normal((trials * T, E))
    idx = oracle.select_topk(l, k).reshape(trials, T * k)
    frac = np.array([len(np.unique(row)) / E for row in idx])
    want = 1 - (1 - k / E) ** T
    # 4-sigma interval; the last term is the resolution of the estimate (one expert in
    # one trial), which matters only where almost every trial touches every expert
    half_width = 4 * frac.std(ddof=1) / math.sqrt(trials) + 1.0 / (E * trials)
    assert abs(frac.mean() - want) <= half_width, (frac.mean(), want)


# ------------------------------------------------------------------ planted mistakes are caught
def _run_pins_on_bruteforce():
    """The brute-force comparison over a few tiny cases; True iff all agree."""
    try:
        for c in CASES[::7]:
            test_oracle_matches_bruteforce(*c)
        test_k_equals_E_softmax_is_dense_mixture()
        test_one_hot_router_is_single_dense_ffn("softmax")
    except AssertionError:
        return False
    return True


MUTANTS = {
    "ties_to_highest_index": ("select_topk", lambda l, k: np.argsort(-l[:, ::-1], 1, kind="stable")[:, :k] * -1 + l.shape[1] - 1),
    "no_renormalisation": ("gate_values", lambda l, i, g: np.take_along_axis(scipy.special.softmax(l, 1), i, 1)),
    "gate_up_swapped": ("swiglu_ffn", lambda v, g, u, dn: (oracle.silu(np.asarray(v) @ np.asarray(u, float).T) * (np.asarray(v) @ np.asarray(g, float).T)) @ np.asarray(dn, float).T),
    "capacity_floor": ("expert_capacity", lambda cf, T, k, E: None if not cf > 0 else int(math.floor(cf * T * k / E))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    import oracle.moe_oracle as mo
    fn_name, fn = MUTANTS[name]
    monkeypatch.setattr(mo, fn_name, fn)
    monkeypatch.setattr(oracle, fn_name, fn, raising=False)
    assert not _run_pins_on_bruteforce(), f"mutant {name} survived the pins"


@pytest.mark.parametrize("case", CASES[::5])
def test_token_outputs_matches_bruteforce(case):
    """The per-token form used at full sizes gives the brute force's outputs for any token
    subset, given that token's routing and kept slots."""
    seed, T, E, d, f, k, gating, cf, integer = case
    x, wr, wg, wu, wd = _tiny_case(seed, T, E, d, f, integer)
    r = _rng(9, seed)
    sh = [(r.standard_normal((2, d)), r.standard_normal((2, d)), r.standard_normal((d, 2)))]
    want = bf.layer(x.tolist(), wr.tolist(), None, wg.tolist(), wu.tolist(), wd.tolist(), k, gating, cf,
                    [tuple(m.tolist() for m in s) for s in sh])
    toks = np.arange(T)[::2]
    got = oracle.token_outputs(x[toks], np.array(want["idx"])[toks], np.array(want["gate"])[toks],
                               np.array(want["kept"])[toks], list(zip(wg, wu, wd)), sh, 1)
    np.testing.assert_allclose(got, np.array(want["y"])[toks], rtol=1e-10, atol=1e-12)
