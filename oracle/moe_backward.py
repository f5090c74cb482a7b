"""Plain CPU oracle of the MoE FFN layer BACKWARD pass (float64, numpy) -- test infrastructure.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU baseline leg of ``bench.py`` may
import or run anything here; the library's GPU path never does and shares no code with it.

What is differentiated: the layer forward of ``moe_oracle`` (router logits, top-k, gates
renormalised over the chosen k, capacity drop, SwiGLU experts, gate-weighted combine, shared
experts), for a loss whose gradient with respect to the layer output y is a given dy, plus
an optional load-balancing loss. Pages: klaylearn.com/glossary/mixture-of-experts and
techbonafide.com "Mixture of Experts (MoE) Explained" (MoE changes training as well as
inference; "Challenges and Tradeoffs": mature implementations add auxiliary losses, as
documented in the Switch Transformer work); shipai.vats.cc "Mixture of Experts (MoE)" (training
adds load-balancing losses so that a few experts do not take every token);
shubhamtatvamasi.com/llm-inference/moe, "Load imbalance" (training adds balancing losses).

Readings (the pages give no formulas for training):
  * The selection (which k experts, which pairs are dropped) is piecewise constant in the
    inputs: no gradient flows through it. The routing decision ``idx`` may be passed in, so
    that a check can use the decision another implementation took on near-tied logits.
  * Load-balancing loss, in the Switch Transformer form the techbonafide page points to:
        L_aux = aux_coef * E * sum_e f_e * P_e,
    f_e = (pairs routed to e before any capacity drop) / (T * k), a constant;
    P_e = mean over tokens of p[t, e], where p is the router's probability over ALL E
    experts: softmax(l) for softmax gating, s / sum(s) with s = sigmoid(l) for sigmoid gating.
  * Every step is the chain rule written out for the forward's formulas, in the forward's
    order; gradients of experts that receive no pairs are zero.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .moe_oracle import (SIGMOID, SOFTMAX, ExpertSource, _expert, _f64, expert_capacity, gate_values,
                         permute, router_logits, select_topk, silu)


def sigmoid(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def silu_grad(a: np.ndarray) -> np.ndarray:
    """d silu(a) / da = s + a s (1 - s), s = sigmoid(a)."""
    s = sigmoid(a)
    return s + a * s * (1.0 - s)


def gate_backward(logits: np.ndarray, idx: np.ndarray, gate: np.ndarray, d_gate: np.ndarray,
                  gating: str) -> np.ndarray:
    """Gradient of the renormalised gates with respect to the logits (dense [T, E], zero off
    the chosen experts).
    softmax: g_j = exp(l_j) / sum_i exp(l_i) over the chosen i, so
        dl_j = g_j (dg_j - sum_i g_i dg_i);
    sigmoid: g_j = s_j / S, S = sum of the chosen s_i, s = sigmoid(l), so
        ds_j = (dg_j - sum_i g_i dg_i) / S and dl_j = ds_j s_j (1 - s_j)."""
    T, E = logits.shape
    inner = (gate * d_gate).sum(axis=1, keepdims=True)
    if gating == SOFTMAX:
        dsel = gate * (d_gate - inner)
    elif gating == SIGMOID:
        s = sigmoid(np.take_along_axis(logits, idx, axis=1))
        S = s.sum(axis=1, keepdims=True)
        dsel = (d_gate - inner) / S * s * (1.0 - s)
    else:
        raise ValueError(f"unknown gating {gating!r}")
    dl = np.zeros((T, E))
    np.put_along_axis(dl, idx, dsel, axis=1)
    return dl


def router_probabilities(logits: np.ndarray, gating: str) -> np.ndarray:
    """p[t, e] over all E experts: softmax(l), or s / sum(s) with s = sigmoid(l)."""
    if gating == SOFTMAX:
        z = np.exp(logits - logits.max(axis=1, keepdims=True))
    else:
        z = sigmoid(logits)
    return z / z.sum(axis=1, keepdims=True)


def aux_loss(logits: np.ndarray, counts: np.ndarray, top_k: int, gating: str, aux_coef: float):
    """L_aux = aux_coef * E * sum_e f_e P_e and its gradient with respect to the logits.
    With F_t = sum_e f_e p[t, e]:
      softmax: dL/dl[t, e] = c p[t, e] (f_e - F_t);
      sigmoid: dL/dl[t, e] = c (f_e - F_t) s_e (1 - s_e) / sum(s)
    with c = aux_coef * E / T."""
    T, E = logits.shape
    f = _f64(counts) / float(T * top_k)
    p = router_probabilities(logits, gating)
    loss = aux_coef * E * float((f * p.mean(axis=0)).sum())
    F = (p * f[None, :]).sum(axis=1, keepdims=True)
    c = aux_coef * E / T
    if gating == SOFTMAX:
        dl = c * p * (f[None, :] - F)
    else:
        s = sigmoid(logits)
        dl = c * (f[None, :] - F) * s * (1.0 - s) / s.sum(axis=1, keepdims=True)
    return loss, dl


def swiglu_backward(v: np.ndarray, wg, wu, wd, dy_rows: np.ndarray):
    """One expert over rows v [m, d] with output gradient dy_rows [m, d]. Forward:
    a = v Wg^T, b = v Wu^T, h = silu(a) b, y = h Wd^T. Returns (y, dv, dWg, dWu, dWd):
      dh = dy Wd; da = dh b silu'(a); db = dh silu(a);
      dWd = dy^T h; dWg = da^T v; dWu = db^T v; dv = da Wg + db Wu."""
    v = _f64(v)
    wg, wu, wd = _f64(wg), _f64(wu), _f64(wd)
    a = v @ wg.T
    b = v @ wu.T
    h = silu(a) * b
    y = h @ wd.T
    dh = dy_rows @ wd
    da = dh * b * silu_grad(a)
    db = dh * silu(a)
    return y, da @ wg + db @ wu, da.T @ v, db.T @ v, dy_rows.T @ h


def backward(x, w_router, bias, dy, *, top_k: int, gating: str, capacity_factor: float,
             experts: ExpertSource, shared: Optional[ExpertSource] = None, n_shared: int = 0,
             aux_coef: float = 0.0, idx: Optional[np.ndarray] = None, want_experts=None) -> dict:
    """Gradients of  sum(y * dy) + L_aux  with respect to every input of the layer.

    Returns dx [T, d], dw_router [E, d], db_router [E], dw_gate / dw_up / dw_down (dicts
    expert -> array, every expert in want_experts (default all), zero for experts without
    pairs), dws_gate / dws_up / dws_down (lists over shared experts), aux_loss, and the
    intermediates d_gate [T, k], dl [T, E], idx, gate, counts, pos."""
    x = _f64(x)
    dy = _f64(dy)
    T, d = x.shape
    E = np.shape(w_router)[0]
    logits = router_logits(x, w_router, bias)
    if idx is None:
        idx = select_topk(logits, top_k)
    idx = np.asarray(idx, np.int64)
    gate = gate_values(logits, idx, gating)
    cap = expert_capacity(capacity_factor, T, top_k, E)
    perm = permute(idx, E, cap)
    keep = (perm["drop"] == 0).reshape(T, top_k)

    dx = np.zeros((T, d))
    d_gate = np.zeros((T, top_k))
    want = range(E) if want_experts is None else want_experts
    dwg, dwu, dwd = {}, {}, {}
    for e in range(E):
        rows_t, rows_j = np.nonzero((idx == e) & keep)  # ascending token
        need = e in want
        if rows_t.size == 0:
            if need:
                wg_, wu_, wd_ = _expert(experts, e)
                dwg[e], dwu[e], dwd[e] = np.zeros_like(wg_), np.zeros_like(wu_), np.zeros_like(wd_)
            continue
        wg_, wu_, wd_ = _expert(experts, e)
        g = gate[rows_t, rows_j][:, None]
        dy_p = g * dy[rows_t]  # y = sum_j g_j y_j: the expert sees g_j dy
        y_e, dv, dwg_e, dwu_e, dwd_e = swiglu_backward(x[rows_t], wg_, wu_, wd_, dy_p)
        d_gate[rows_t, rows_j] = (dy[rows_t] * y_e).sum(axis=1)
        np.add.at(dx, rows_t, dv)
        if need:
            dwg[e], dwu[e], dwd[e] = dwg_e, dwu_e, dwd_e
    dws_g, dws_u, dws_d = [], [], []
    for s in range(n_shared):
        _, dv, a_, b_, c_ = swiglu_backward(x, *_expert(shared, s), dy)
        dx += dv
        dws_g.append(a_)
        dws_u.append(b_)
        dws_d.append(c_)
    dl = gate_backward(logits, idx, gate, d_gate, gating)
    loss = 0.0
    if aux_coef != 0.0:
        loss, dl_aux = aux_loss(logits, perm["counts"], top_k, gating, aux_coef)
        dl = dl + dl_aux
    wr = _f64(w_router)
    dx += dl @ wr
    return dict(dx=dx, dw_router=dl.T @ x, db_router=dl.sum(axis=0), dw_gate=dwg, dw_up=dwu, dw_down=dwd,
                dws_gate=dws_g, dws_up=dws_u, dws_down=dws_d, aux_loss=loss, d_gate=d_gate, dl=dl, idx=idx,
                gate=gate, counts=perm["counts"], pos=perm["pos"], logits=logits)
