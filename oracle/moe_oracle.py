"""Plain CPU oracle of the Mixture-of-Experts FFN layer forward (float64, numpy).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or run anything in this package; the library's
GPU path never does, and shares no code with it.

Every step below is the plain definition written out, one library primitive (a matrix
product, a stable sort, a bincount) at a time, with no blocking or fusion. All arithmetic
is float64 on the exact stored input values (bfloat16 and float32 inputs widen exactly).

Sources (the pages this follows):
  * shubhamtatvamasi.com/llm-inference/moe, "Mixture of Experts": section "The router"
    (one linear layer scores every expert; softmax, or a sigmoid as in DeepSeek-V3, then
    the chosen gates renormalised to sum to one; shared experts every token visits),
    section "Load imbalance" (capacity factor x ideal tokens, overflow skips the expert
    and stays on the residual path; dropless), and the Q&A entries "How does a top-k
    router work?" and "What are capacity factor and token dropping ..." (limit
    factor x (T.k/E); output = gate-weighted sum of the chosen experts' outputs).
  * shipai.vats.cc/learn/advanced-concepts/mixture-of-experts, "Mixture of Experts (MoE)":
    section "How routing works (intuition)" (score N experts, take top-k, run them,
    combine with router weights).
  * klaylearn.com/glossary/mixture-of-experts, "Mixture of Experts": the definition
    paragraph on the distributed layer (permute tokens by destination expert, grouped
    GEMM per expert batch, undo the permutation).
  * techbonafide.com "Mixture of Experts (MoE) Explained": section "Experts as Specialized
    Subnetworks" (an expert is a standard feed-forward block).

Readings where the pages are silent (each is listed with its reason in the design notes):
  selection is made on the logits (bias included) -- equivalent to selecting on softmax or
  sigmoid scores, which are monotone; ties go to the lower expert index; gates are
  renormalised over the chosen k for both gatings; capacity C = ceil(cf * T * k / E)
  evaluated in float64 from the float32 factor, cf <= 0 meaning dropless; the kept tokens
  of an over-full expert are those with the lowest token index; a dropped slot adds
  nothing and the other gates are not renormalised; the residual add is outside the
  layer; each shared expert is added with weight one; an expert is the SwiGLU block
  (silu(v Wg) * (v Wu)) Wd without biases.

Weight layout (out-features-major): router [E][d]; gate, up [E][f][d]; down [E][d][f].
The products are v . Wg^T etc., i.e. the row-vector y = x . W of the d x f matrices.

FP8 expert weights (shubhamtatvamasi.com, "Memory vs compute, quantified": FP8 halves the
weight bytes of BF16; shipai.vats.cc, "Production reality: serving MoE is not free":
quantisation error differs per expert). The pages fix no format; the reading taken is OCP
E4M3 codes with one scale per output row of each expert matrix. ``e4m3_value`` decodes
the format from its definition and ``dequantize_rows`` applies the scales; the grouped MLP
then runs on those exact values, so an FP8 layer is the plain layer on dequantised
weights.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Union

import numpy as np

SOFTMAX = "softmax"
SIGMOID = "sigmoid"

ExpertSource = Union[Callable[[int], Sequence[np.ndarray]], Sequence[Sequence[np.ndarray]]]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _expert(src: ExpertSource, e: int):
    w = src(e) if callable(src) else src[e]
    return tuple(_f64(m) for m in w)


# ---------------------------------------------------------------- step 1: router
def router_logits(x, w_router, bias=None) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * W_r[e, i] + b[e]  ("The router": one linear layer that
    scores the token's hidden vector against every expert)."""
    logits = _f64(x) @ _f64(w_router).T
    if bias is not None:
        logits = logits + _f64(bias)[None, :]
    return logits


# ---------------------------------------------------------------- step 2: top-k
def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """The k highest-scoring experts per token, ordered by descending logit, ties to the
    lower expert index (the router retains the k best). Returns int64 [T, k]."""
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # a stable sort of -l keeps equal logits in ascending expert order
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


# ---------------------------------------------------------------- step 3: gates
def gate_values(logits: np.ndarray, idx: np.ndarray, gating: str) -> np.ndarray:
    """Gate of each chosen expert, renormalised over the chosen k to sum to one.

    softmax: exp(l_j - m) / sum over chosen exp(l_i - m), m the largest chosen logit;
    this equals the softmax over all E renormalised over the chosen k (the common
    denominator cancels). sigmoid (DeepSeek-V3 style): s_j / sum over chosen s_i with
    s = 1 / (1 + exp(-l))."""
    sel = np.take_along_axis(logits, idx, axis=1)
    if gating == SOFTMAX:
        m = sel.max(axis=1, keepdims=True)
        p = np.exp(sel - m)
    elif gating == SIGMOID:
        with np.errstate(over="ignore"):
            p = 1.0 / (1.0 + np.exp(-sel))
    else:
        raise ValueError(f"unknown gating {gating!r}")
    return p / p.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k: int, gating: str):
    """Steps 1-3. Returns (topk_idx int64 [T,k], topk_gate f64 [T,k], logits f64 [T,E])."""
    logits = router_logits(x, w_router, bias)
    idx = select_topk(logits, k)
    return idx, gate_values(logits, idx, gating), logits


# ---------------------------------------------------------------- step 4: capacity
def expert_capacity(capacity_factor: float, T: int, k: int, E: int) -> Optional[int]:
    """Per-expert limit factor x (T.k/E), rounded up; None when dropless (factor <= 0).
    The factor is the float32 the caller passes, evaluated in float64 as cf * (T*k) / E."""
    cf = float(np.float32(capacity_factor))
    if not cf > 0:
        return None
    return int(math.ceil(cf * float(T * k) / float(E)))


# ---------------------------------------------------------------- step 5: permutation
def permute(idx: np.ndarray, n_experts: int, capacity: Optional[int] = None) -> dict:
    """Group the (token, slot) pairs by destination expert.

    A pair is identified by s = t*k + j. Pairs are ordered by expert, then by ascending
    token (each token chooses an expert at most once, so ascending s is ascending t).
    With a capacity C, the first C pairs of each expert are kept and the rest dropped.
    Returns counts[E] (before dropping), offsets[E+1] (after), sorted_slot[N_kept],
    pos[T*k] (index in the grouped order, -1 when dropped) and drop[T*k] (uint8)."""
    T, k = idx.shape
    E = n_experts
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    first = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rank = np.empty(T * k, np.int64)
    rank[order] = np.arange(T * k, dtype=np.int64) - first[flat[order]]
    keep = np.ones(T * k, bool) if capacity is None else rank < capacity
    kept = counts if capacity is None else np.minimum(counts, capacity)
    offsets = np.concatenate([[0], np.cumsum(kept)]).astype(np.int64)
    pos = np.where(keep, offsets[flat] + rank, -1).astype(np.int64)
    sorted_slot = order[keep[order]].astype(np.int64)
    return dict(counts=counts, offsets=offsets, sorted_slot=sorted_slot, pos=pos,
                drop=(~keep).astype(np.uint8))


# ---------------------------------------------------------------- step 6: experts
def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a)."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_ffn(v, w_gate, w_up, w_down) -> np.ndarray:
    """One expert: (silu(v . Wg) * (v . Wu)) . Wd for rows v [m, d] (stored weights are
    Wg^T, Wu^T [f, d] and Wd^T [d, f])."""
    v = _f64(v)
    h = silu(v @ _f64(w_gate).T) * (v @ _f64(w_up).T)
    return h @ _f64(w_down).T


def grouped_mlp(x, sorted_slot, offsets, k: int, experts: ExpertSource) -> np.ndarray:
    """Each expert's FFN over its batch of gathered token rows, in the grouped order:
    y_perm[p] = FFN_e(x[sorted_slot[p] // k]) for offsets[e] <= p < offsets[e+1]."""
    x = _f64(x)
    E = len(offsets) - 1
    y_perm = np.zeros((int(offsets[E]), x.shape[1]))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        y_perm[a:b] = swiglu_ffn(x[np.asarray(sorted_slot[a:b]) // k], *_expert(experts, e))
    return y_perm


def shared_mlp(x, shared: ExpertSource, n_shared: int) -> np.ndarray:
    """Every shared expert's FFN over all tokens: [n_shared, T, d]."""
    return np.stack([swiglu_ffn(x, *_expert(shared, s)) for s in range(n_shared)])


# ---------------------------------------------------------------- FP8 expert weights
def e4m3_value(codes) -> np.ndarray:
    """The real number each OCP FP8 E4M3 code denotes, in float64 (exact).

    Byte = sign bit | 4-bit exponent field E | 3-bit mantissa field M, exponent bias 7:
      E == 0:            (-1)^s * 2^-6 * M/8        (zero and subnormals)
      E in 1..15:        (-1)^s * 2^(E-7) * (1 + M/8)
    except E == 15 with M == 7 (0x7F, 0xFF), which is NaN; the format has no infinities,
    so 0x7E = 2^8 * 1.75 = 448 is the largest value. (Pages: shubhamtatvamasi.com, "Memory
    vs compute, quantified": FP8 weights take one byte per parameter.)"""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    neg = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(neg == 1, -mag, mag)


def dequantize_rows(codes, scale) -> np.ndarray:
    """W[n, i] = scale[n] * e4m3(code[n, i]): one scale per output row (stored row)."""
    return _f64(scale)[:, None] * e4m3_value(codes)


def fp8_expert(codes_gate, codes_up, codes_down, scale_gate, scale_up, scale_down):
    """The exact weight values (gate, up, down) of one FP8 expert, for swiglu_ffn."""
    return (dequantize_rows(codes_gate, scale_gate), dequantize_rows(codes_up, scale_up),
            dequantize_rows(codes_down, scale_down))


# ---------------------------------------------------------------- step 7: combine
def combine(y_perm: np.ndarray, pos: np.ndarray, gate: np.ndarray,
            y_shared: Optional[np.ndarray] = None) -> np.ndarray:
    """Undo the permutation and take the gate-weighted sum:
    y[t] = sum over kept j of gate[t, j] * y_perm[pos[t, j]]  (+ every shared output)."""
    T, k = gate.shape
    pos = np.asarray(pos).reshape(T, k)
    y = np.zeros((T, y_perm.shape[1]))
    for j in range(k):
        p = pos[:, j]
        m = p >= 0
        y[m] += gate[m, j, None] * y_perm[p[m]]
    if y_shared is not None:
        y += np.asarray(y_shared, np.float64).sum(axis=0)
    return y


# ---------------------------------------------------------------- whole layer
def forward(x, w_router, bias, *, top_k: int, gating: str, capacity_factor: float,
            experts: ExpertSource, shared: Optional[ExpertSource] = None,
            n_shared: int = 0) -> dict:
    """Steps 1-7 on all T tokens; returns every stage's result."""
    T = np.shape(x)[0]
    E = np.shape(w_router)[0]
    idx, gate, logits = route(x, w_router, bias, top_k, gating)
    cap = expert_capacity(capacity_factor, T, top_k, E)
    perm = permute(idx, E, cap)
    y_perm = grouped_mlp(x, perm["sorted_slot"], perm["offsets"], top_k, experts)
    y_shared = shared_mlp(x, shared, n_shared) if n_shared > 0 else None
    y = combine(y_perm, perm["pos"], gate, y_shared)
    return dict(logits=logits, idx=idx, gate=gate, capacity=cap, y_perm=y_perm,
                y_shared=y_shared, y=y, **perm)


def token_outputs(x_rows, idx_rows, gate_rows, keep_rows, experts: ExpertSource,
                  shared: Optional[ExpertSource] = None, n_shared: int = 0) -> np.ndarray:
    """Step 6-7 for a subset of tokens, given their routing and which of their slots are
    kept: y = sum over kept j of gate_j * FFN_{idx_j}(x) + shared outputs. Each expert's
    weights are widened once for all rows that chose it."""
    x_rows = _f64(x_rows)
    n, k = np.shape(idx_rows)
    y = np.zeros((n, x_rows.shape[1]))
    for e in np.unique(np.asarray(idx_rows)[np.asarray(keep_rows, bool)]):
        w = _expert(experts, int(e))
        for j in range(k):
            m = (np.asarray(idx_rows)[:, j] == e) & np.asarray(keep_rows, bool)[:, j]
            if m.any():
                y[m] += np.asarray(gate_rows, np.float64)[m, j, None] * swiglu_ffn(x_rows[m], *w)
    if n_shared > 0:
        y += shared_mlp(x_rows, shared, n_shared).sum(axis=0)
    return y
