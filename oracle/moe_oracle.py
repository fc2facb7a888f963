"""CPU oracle for the sparsely-gated noisy top-k Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import or call this module.  The product path never
routes through it, and it shares no code with the HIP implementation: it takes
plain numpy arrays and computes, in float64, what the pages define, one step
after the other, with no blocking, fusion or reordering.

Pages cited (titles as published):
  [MoE lesson]  "MoE:稀疏门控混合专家" (nengyongai.cn lesson on Shazeer et al.
                2017): section 二 (what one MoE layer looks like: the 512 ->
                1024 -> 512 expert FFN and y = sum_i G(x)_i E_i(x)), section 三
                (how the gate picks: score table W_g, KeepTopK to -inf, softmax,
                the worked 8-expert top-2 example, the 16 x 256 "-h"
                hierarchy), section 四 (noise: H = x W_g + noise * softplus(x
                W_noise), noise redrawn every call).
  [Paper card]  "Outrageously Large Neural Networks: The Sparsely-Gated
                Mixture-of-Experts Layer - 中文验证版" (ai-papers.xuzou.cn):
                section 瓶颈 (each expert receives about k*b/n rows), section
                方法适配 (k = 4 in many LM runs; importance and load losses keep
                rows spread over experts).
  [Reading note] "Outrageously Large Neural Networks — MoE 怎样让模型“很大但
                不每次全算”" (wudongming97.github.io): sections 核心想法 and
                方法怎么做 (top-k gating, learnable noise, importance loss on
                per-expert gate totals and load loss on per-expert row counts).
  [Mixtral page] "MoE 混合专家：参数大、计算省" (transformer.xph.ink), section
                核心概念 (Mixtral: 8 experts, top-2 routing).

Readings of points the pages leave open (each also listed with its reason in
the design notes):
  * top-k ties go to the lower expert index; the k kept experts of a token are
    stored in ascending expert index ("slot" order);
  * softplus is exact, with no added floor;
  * the noise draw eps ~ N(0,1) is an input; no eps means noise-free gating;
  * the importance of expert e is the sum over tokens of its gate; the load of
    expert e is the sum over tokens of the probability that e would still be
    in the top-k if only its own noise were redrawn, Phi((clean - theta) /
    softplus(raw)) with theta the k-th largest noisy logit among the other
    experts; CV^2 is population variance over squared mean (0 when the mean
    is 0); without noise the load is the hard row count;
  * the hierarchy multiplies the primary (group) gate by the secondary
    (expert-in-group) gate; each group has its own secondary tables, which are
    the rows g*Eg .. (g+1)*Eg-1 of the flat [E][d] tables;
  * the SwiGLU expert is (silu(X W_gate) * (X W_up)) W_down, no biases.
  * parity unpinned: the hierarchical load (reported as hard counts per
    expert) has no page formula.
  * backward pass: the objective is sum(dy * y) + w_imp CV^2(Importance) +
    w_load CV^2(Load); the kept set and the experts ranked k-th and (k+1)-th
    are held fixed (the choice itself has no gradient), so the threshold
    theta of the smooth load passes its gradient to the score of the expert
    it was read from; noise-free gating and the hierarchy have a hard load
    and no load gradient; in the hierarchy the product of the two levels'
    gates passes its gradient to each level, which then differentiates like
    a flat gate over its kept scores.

Array layouts follow the library's: x [T][d]; w_gate, w_noise [E][d] (the
pages' d x n table stored transposed); w1 [E][h][d]; w3 [E][h][d]; w2 [E][d][h].
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
from scipy.special import erfc


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (bf16 is up-cast exactly)
        a = a.detach().to("cpu").float().numpy()
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Scalar functions
# ---------------------------------------------------------------------------

def softplus(z: np.ndarray) -> np.ndarray:
    """softplus(z) = ln(1 + e^z), written in the overflow-safe form
    max(z, 0) + ln(1 + e^-|z|).  [MoE lesson, section 四: the noise scale]"""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def normal_cdf(z: np.ndarray) -> np.ndarray:
    """Standard normal CDF, Phi(z) = erfc(-z / sqrt 2) / 2."""
    return 0.5 * erfc(-np.asarray(z, dtype=np.float64) / math.sqrt(2.0))


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z), the gate nonlinearity of the
    SwiGLU expert; sigmoid is written (1 + tanh(z/2)) / 2 so that no
    exponential overflows."""
    z = np.asarray(z, dtype=np.float64)
    return z * (0.5 * (1.0 + np.tanh(0.5 * z)))


# ---------------------------------------------------------------------------
# Gating  [MoE lesson, sections 三 and 四]
# ---------------------------------------------------------------------------

def noisy_logits(x, w_gate, w_noise=None, bias=None, eps=None):
    """Scores of every expert for every token.

    clean = x W_g (+ bias), one score per expert column of the table;
    with noise: H = clean + eps * softplus(x W_noise); without: H = clean.
    Returns (clean, sp, H); sp is None without noise.
    [MoE lesson, section 三 (score table) and section 四 (the noisy score)]
    """
    x = _f64(x)
    clean = x @ _f64(w_gate).T
    if bias is not None:
        clean = clean + _f64(bias)[None, :]
    if eps is None or w_noise is None:
        return clean, None, clean.copy()
    sp = softplus(x @ _f64(w_noise).T)
    H = clean + _f64(eps) * sp
    return clean, sp, H


def keep_top_k(H: np.ndarray, k: int):
    """KeepTopK: per token, the k largest scores survive, the rest become -inf.

    Ties are broken toward the lower expert index (a stable sort of the
    negated scores keeps equal scores in index order).  Returns
      idx    [T][k] int32, the kept experts in ascending index order,
      kth    [T]  the k-th largest score,
      k1th   [T]  the (k+1)-th largest score (-inf if k == E),
      margin [T]  kth - k1th.
    [MoE lesson, section 三, step 2]
    """
    H = np.asarray(H, dtype=np.float64)
    T, E = H.shape
    order = np.argsort(-H, axis=1, kind="stable")
    kept = order[:, :k]
    idx = np.sort(kept, axis=1).astype(np.int32)
    rows = np.arange(T)
    kth = H[rows, order[:, k - 1]] if T else np.zeros(0)
    if k < E:
        k1th = H[rows, order[:, k]] if T else np.zeros(0)
    else:
        k1th = np.full(T, -np.inf)
    with np.errstate(invalid="ignore"):
        margin = kth - k1th
    return idx, kth, k1th, margin


def kept_softmax(H: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over the kept scores only; the dropped ones are -inf and their
    exponential is 0.  Returns gates [T][k] in the slot order of idx.
    [MoE lesson, section 三, step 3]"""
    H = np.asarray(H, dtype=np.float64)
    kept = np.take_along_axis(H, idx.astype(np.int64), axis=1)
    if kept.shape[0] == 0:
        return kept
    m = kept.max(axis=1, keepdims=True)
    w = np.exp(kept - m)
    return w / w.sum(axis=1, keepdims=True)


def dense_gates(idx: np.ndarray, gates: np.ndarray, n_experts: int) -> np.ndarray:
    """The sparse gate vector G(x) as a dense [T][E] array, zero off the kept set."""
    T = idx.shape[0]
    G = np.zeros((T, n_experts), dtype=np.float64)
    for s in range(idx.shape[1]):
        G[np.arange(T), idx[:, s]] = gates[:, s]
    return G


def flat_gate(x, w_gate, w_noise, bias, eps, k):
    """Noisy top-k gate of the flat layer.  Returns a dict with clean, sp, H,
    idx, gates, kth, k1th, margin."""
    clean, sp, H = noisy_logits(x, w_gate, w_noise, bias, eps)
    idx, kth, k1th, margin = keep_top_k(H, k)
    gates = kept_softmax(H, idx)
    return dict(clean=clean, sp=sp, H=H, idx=idx, gates=gates,
                kth=kth, k1th=k1th, margin=margin)


def hier_gate(x, w_gate_p, w_noise_p, eps_p, w_gate, w_noise, eps,
              n_groups, k_groups, k_per_group):
    """Two-level gate of the "-h" layer: the primary gate keeps k_groups of the
    n_groups groups, then inside each kept group a secondary gate keeps
    k_per_group of its experts; the final gate is the product of the two
    levels' gates.  Expert j of group g is global expert g*Eg + j.
    [MoE lesson, section 三: 16 groups x 256 experts, 2 groups then 2 experts]
    The product rule is a reading (the page gives only the selection rule).
    Returns idx [T][k] (ascending expert index), gates [T][k], the primary
    gate's dict, and margin [T] = the smallest margin over both levels.
    """
    x = _f64(x)
    T = x.shape[0]
    E = _f64(w_gate).shape[0]
    Eg = E // n_groups
    prim = flat_gate(x, w_gate_p, w_noise_p, None, eps_p, k_groups)
    k = k_groups * k_per_group
    idx = np.zeros((T, k), dtype=np.int32)
    gates = np.zeros((T, k), dtype=np.float64)
    margin = prim["margin"].copy()
    wg = _f64(w_gate)
    wn = _f64(w_noise) if w_noise is not None else None
    ep = _f64(eps) if eps is not None else None
    for t in range(T):
        s = 0
        for a in range(k_groups):          # groups in ascending order
            g = int(prim["idx"][t, a])
            rows = slice(g * Eg, (g + 1) * Eg)
            sub = flat_gate(x[t:t + 1], wg[rows], None if wn is None else wn[rows],
                            None, None if ep is None else ep[t:t + 1, g, :],
                            k_per_group)
            margin[t] = min(margin[t], sub["margin"][0])
            for b in range(k_per_group):   # experts in ascending order
                idx[t, s] = g * Eg + sub["idx"][0, b]
                gates[t, s] = prim["gates"][t, a] * sub["gates"][0, b]
                s += 1
    return dict(idx=idx, gates=gates, margin=margin, primary=prim)


# ---------------------------------------------------------------------------
# Routing: group the (token, slot) pairs by expert  [Paper card, section 瓶颈]
# ---------------------------------------------------------------------------

def route(idx: np.ndarray, n_experts: int, capacity: int = 0):
    """Stable grouping of the T*k (token, slot) assignments by expert.

    counts[e]  number of assignments to expert e (kept ones, with a capacity);
    offsets    exclusive prefix sum of counts, length E+1;
    perm[p]    the assignment t*k+s placed at position p: expert-contiguous,
               tokens ascending inside each expert (length offsets[E]);
    inv[t*k+s] the position p of that assignment (inverse of perm), or -1.

    With capacity > 0 an expert keeps only the first `capacity` assignments
    that reach it in token order; the later ones are dropped (inv = -1).
    [Mixtral page, section 核心概念: a per-expert buffer limit, overflow dropped]
    """
    T, k = idx.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in idx.reshape(-1):
        if capacity <= 0 or counts[e] < capacity:
            counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    perm = np.zeros(int(offsets[-1]), dtype=np.int64)
    inv = np.full(T * k, -1, dtype=np.int64)
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            if fill[e] == offsets[e + 1]:
                continue  # expert e is full
            p = fill[e]
            fill[e] += 1
            perm[p] = t * k + s
            inv[t * k + s] = p
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))


# ---------------------------------------------------------------------------
# Experts  [MoE lesson, section 二: a one-hidden-layer FFN, 512 -> 1024 -> 512]
# ---------------------------------------------------------------------------

def expert_relu(X, w1_e, w2_e) -> np.ndarray:
    """E(X) = max(X W1, 0) W2 with W1 stored [h][d] and W2 stored [d][h]."""
    X = _f64(X)
    hid = np.maximum(X @ _f64(w1_e).T, 0.0)
    return hid @ _f64(w2_e).T


def expert_swiglu(X, w1_e, w3_e, w2_e) -> np.ndarray:
    """E(X) = (silu(X W_gate) * (X W_up)) W_down, with W_gate = w1 [h][d],
    W_up = w3 [h][d], W_down = w2 [d][h].  [Mixtral page, section 核心概念]"""
    X = _f64(X)
    hid = silu(X @ _f64(w1_e).T) * (X @ _f64(w3_e).T)
    return hid @ _f64(w2_e).T


def expert_apply(X, e, w1, w2, w3=None) -> np.ndarray:
    if w3 is None:
        return expert_relu(X, w1[e], w2[e])
    return expert_swiglu(X, w1[e], w3[e], w2[e])


def run_experts(x, perm, offsets, k, w1, w2, w3=None) -> np.ndarray:
    """y_sorted[p] = E_e(x[perm[p] // k]) for every position p of expert e.
    Experts with no rows are not evaluated (their gate is zero for every
    token).  [MoE lesson, section 二: dropped experts are skipped]"""
    x = _f64(x)
    E = len(offsets) - 1
    A = int(offsets[-1])
    d = x.shape[1]
    y_sorted = np.zeros((A, _f64(w2[0]).shape[0] if E else d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = perm[lo:hi] // k
        y_sorted[lo:hi] = expert_apply(x[toks], e, w1, w2, w3)
    return y_sorted


def combine(y_sorted, inv, gates) -> np.ndarray:
    """y_t = sum over slots s of gate[t,s] * y_sorted[inv[t*k+s]], slots in
    ascending order; a slot dropped by a capacity (inv = -1) adds nothing.
    [MoE lesson, section 二: y = sum_i G(x)_i E_i(x)]"""
    gates = np.asarray(gates, dtype=np.float64)
    T, k = gates.shape
    d = y_sorted.shape[1] if y_sorted.ndim == 2 else 0
    y = np.zeros((T, d))
    inv2 = np.asarray(inv).reshape(T, k)
    for s in range(k):
        kept = inv2[:, s] >= 0
        y[kept] += gates[kept, s:s + 1] * y_sorted[inv2[kept, s]]
    return y


# ---------------------------------------------------------------------------
# Balance statistics  [Reading note, sections 核心想法/方法怎么做; Paper card,
# section 方法适配]
# ---------------------------------------------------------------------------

def cv_squared(v) -> float:
    """Squared coefficient of variation: population variance / mean^2
    (0 for an all-zero vector)."""
    v = np.asarray(v, dtype=np.float64)
    if v.size == 0:
        return 0.0
    m = v.mean()
    if m == 0.0:
        return 0.0
    return float(((v - m) ** 2).mean() / (m * m))


def importance(idx, gates, n_experts) -> np.ndarray:
    """Importance_e = sum over tokens of G(x)_e."""
    return dense_gates(idx, gates, n_experts).sum(axis=0)


def load_estimate(clean, sp, H, idx, kth, k1th) -> np.ndarray:
    """Smooth load: Load_e = sum_t P(e in top-k of token t when only expert e's
    noise is redrawn) = sum_t Phi((clean[t,e] - theta[t,e]) / sp[t,e]),
    theta[t,e] = k-th largest noisy score among the experts other than e,
    which is the (k+1)-th largest score if e is kept and the k-th otherwise.
    """
    T, E = H.shape
    kept = np.zeros((T, E), dtype=bool)
    for s in range(idx.shape[1]):
        kept[np.arange(T), idx[:, s]] = True
    theta = np.where(kept, k1th[:, None], kth[:, None])
    return normal_cdf((clean - theta) / sp).sum(axis=0)


def balance_stats(n_experts, idx, gates, counts, gate_info=None,
                  w_importance=1.0, w_load=1.0):
    """importance[E], load[E], cv2 of each, and the weighted loss.

    gate_info is the flat gate's dict when the smooth load applies (flat noisy
    gating); otherwise the load is the hard row count of each expert.
    """
    imp = importance(idx, gates, n_experts)
    if gate_info is not None and gate_info.get("sp") is not None:
        load = load_estimate(gate_info["clean"], gate_info["sp"], gate_info["H"],
                             gate_info["idx"], gate_info["kth"], gate_info["k1th"])
    else:
        load = np.asarray(counts, dtype=np.float64)
    ci, cl = cv_squared(imp), cv_squared(load)
    return dict(importance=imp, load=load, cv2_importance=ci, cv2_load=cl,
                loss=w_importance * ci + w_load * cl)


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------

def gate(inp: Dict, cfg) -> Dict:
    """Flat or hierarchical gate, chosen by cfg.n_groups."""
    if cfg.n_groups:
        return hier_gate(inp["x"], inp["w_gate_p"], inp.get("w_noise_p"),
                         inp.get("eps_p"), inp["w_gate"], inp.get("w_noise"),
                         inp.get("eps"), cfg.n_groups, cfg.k_groups,
                         cfg.k_per_group)
    return flat_gate(inp["x"], inp["w_gate"], inp.get("w_noise"), inp.get("bias"),
                     inp.get("eps"), cfg.top_k)


def forward(inp: Dict, cfg, w_importance=1.0, w_load=1.0,
            with_experts: bool = True) -> Dict:
    """Whole layer: gate -> route -> experts -> combine -> balance stats.
    Returns every intermediate the HIP path exposes."""
    g = gate(inp, cfg)
    idx, gates = g["idx"], g["gates"]
    capacity = getattr(cfg, "capacity", 0)
    counts, offsets, perm, inv = route(idx, cfg.n_experts, capacity)
    out = dict(idx=idx, gates=gates, margin=g["margin"], counts=counts,
               offsets=offsets, perm=perm, inv=inv, gate_info=g)
    # the balance statistics describe the gate's choice, before any drop
    gate_counts = route(idx, cfg.n_experts)[0] if capacity > 0 else counts
    if with_experts:
        w1 = _f64(inp["w1"])
        w2 = _f64(inp["w2"])
        w3 = _f64(inp.get("w3"))
        y_sorted = run_experts(inp["x"], perm, offsets, cfg.top_k, w1, w2, w3)
        out["y_sorted"] = y_sorted
        out["y"] = combine(y_sorted, inv, gates)
    out.update(balance_stats(cfg.n_experts, idx, gates, gate_counts,
                             None if cfg.n_groups else g, w_importance, w_load))
    return out


# ---------------------------------------------------------------------------
# Per-batch equal-size expert mask and its inference thresholds  [Paper card,
# section 方法适配: in some translation runs a per-batch mask gives every
# expert the same batch size during training, and per-expert thresholds
# approximate that mask at inference]
#
# Readings of what the page leaves open (each also in the design notes):
#   * batch mask: expert e keeps the m tokens of the batch with the largest
#     scores H[:, e] (ties: the lower token index), m given by the caller
#     (m = k T / E gives every token k experts on average);
#   * threshold mask: token t is kept by expert e iff H[t, e] >= theta[e]
#     (theta set to each expert's m-th largest score over a batch reproduces
#     that batch's mask when the scores have no ties);
#   * a token's gates are the softmax over the scores of the experts that
#     kept it (the lesson page's softmax over the kept scores), zero
#     elsewhere; a token kept by no expert has no gates and y = 0;
#   * rows: expert e takes its kept tokens in ascending token order, at most
#     `capacity` of them (0: no limit); later ones are dropped and add
#     nothing to y, the gates are not renormalised (as with the capacity of
#     the top-k layer);
#   * balance statistics: importance as in the top-k layer (sum of each
#     expert's gates over the batch, before any drop), load = the hard count
#     of kept tokens per expert before any drop.
# ---------------------------------------------------------------------------

def batch_mask(H: np.ndarray, m: int) -> np.ndarray:
    """[T][E] bool: expert e keeps the m best tokens of its column of H."""
    H = np.asarray(H, dtype=np.float64)
    T, E = H.shape
    keep = np.zeros((T, E), dtype=bool)
    for e in range(E):
        order = np.argsort(-H[:, e], kind="stable")   # ties: lower token first
        keep[order[:min(m, T)], e] = True
    return keep


def threshold_mask(H: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """[T][E] bool: H[t, e] >= theta[e]."""
    return np.asarray(H, dtype=np.float64) >= np.asarray(theta, dtype=np.float64)[None, :]


def masked_gates(H: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """[T][E] gates: per token, the softmax over its kept scores."""
    H = np.asarray(H, dtype=np.float64)
    G = np.zeros_like(H)
    for t in range(H.shape[0]):
        kept = np.nonzero(keep[t])[0]
        if kept.size == 0:
            continue
        h = H[t, kept]
        w = np.exp(h - h.max())
        G[t, kept] = w / w.sum()
    return G


def masked_route(keep: np.ndarray, capacity: int = 0):
    """Rows of each expert from a keep mask: counts[E], offsets[E+1],
    perm[p] = the token at position p (expert-contiguous, tokens ascending),
    and pos[T][E] = the position of (t, e), or -1 when e did not keep t or
    its capacity dropped it."""
    T, E = keep.shape
    counts = np.zeros(E, dtype=np.int64)
    pos = np.full((T, E), -1, dtype=np.int64)
    cols = []
    for e in range(E):
        toks = np.nonzero(keep[:, e])[0]           # ascending
        if capacity > 0:
            toks = toks[:capacity]
        counts[e] = toks.size
        cols.append(toks)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.zeros(int(offsets[-1]), dtype=np.int64)
    for e in range(E):
        p = offsets[e] + np.arange(cols[e].size)
        perm[p] = cols[e]
        pos[cols[e], e] = p
    return counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32), pos


def masked_forward(inp: Dict, cfg, rows_per_expert: int = 0, thresholds=None,
                   w_importance=1.0, w_load=1.0) -> Dict:
    """The flat layer with the batch mask (rows_per_expert = m > 0) or the
    threshold mask (thresholds [E]) in place of KeepTopK; cfg.capacity caps
    the rows of an expert.  Returns the mask, gates [T][E], routing, y and
    the balance statistics."""
    clean, sp, H = noisy_logits(inp["x"], inp["w_gate"], inp.get("w_noise"), inp.get("bias"),
                                inp.get("eps"))
    if thresholds is None:
        keep = batch_mask(H, rows_per_expert)
    else:
        keep = threshold_mask(H, thresholds)
    G = masked_gates(H, keep)
    counts, offsets, perm, pos = masked_route(keep, getattr(cfg, "capacity", 0))
    x = _f64(inp["x"])
    w1, w2, w3 = _f64(inp["w1"]), _f64(inp["w2"]), _f64(inp.get("w3"))
    E = cfg.n_experts
    y_sorted = np.zeros((int(offsets[-1]), x.shape[1]))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y_sorted[lo:hi] = expert_apply(x[perm[lo:hi]], e, w1, w2, w3)
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        for e in np.nonzero(pos[t] >= 0)[0]:         # experts ascending
            y[t] += G[t, e] * y_sorted[pos[t, e]]
    imp = G.sum(axis=0)
    load = keep.sum(axis=0).astype(np.float64)
    ci, cl = cv_squared(imp), cv_squared(load)
    return dict(H=H, keep=keep, gates=G, counts=counts, offsets=offsets, perm=perm, pos=pos,
                y_sorted=y_sorted, y=y, importance=imp, load=load, cv2_importance=ci,
                cv2_load=cl, loss=w_importance * ci + w_load * cl)


def dense_forward(inp: Dict, cfg) -> np.ndarray:
    """Brute force: evaluate every expert on every token and sum with the dense
    gate vector, y_t = sum over all e of G(x_t)_e E_e(x_t).  Tiny inputs only.
    [MoE lesson, section 二]"""
    g = gate(inp, cfg)
    G = dense_gates(g["idx"], g["gates"], cfg.n_experts)
    x = _f64(inp["x"])
    w1, w2, w3 = _f64(inp["w1"]), _f64(inp["w2"]), _f64(inp.get("w3"))
    y = np.zeros((x.shape[0], w2.shape[1]))
    for e in range(cfg.n_experts):
        y += G[:, e:e + 1] * expert_apply(x, e, w1, w2, w3)
    return y


# ---------------------------------------------------------------------------
# Backward pass  [Reading note, sections 问题是什么 and 方法怎么做; Paper card,
# sections 瓶颈 and 方法适配; Mixtral page, section 核心概念]
#
# The objective is L = sum(dy * y) + w_imp * CV^2(Importance) + w_load *
# CV^2(Load): dy is the gradient that flows into the layer output from above,
# and the two balance losses are added to the training objective with the
# caller's weights.  The choice of the kept experts is a discrete step with no
# gradient (the reading note's point that a hard choice is not
# differentiable): the kept set, and which expert holds the k-th and (k+1)-th
# score, are held fixed, and gradients flow through the softmax weights of the
# kept scores, the noisy scores, the smooth load estimate and the experts.
# Hidden activations are recomputed from the inputs (the paper card's
# activation recomputation) rather than saved.
# ---------------------------------------------------------------------------

def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def normal_pdf(z):
    """phi(z) = exp(-z^2 / 2) / sqrt(2 pi), the derivative of Phi."""
    z = np.asarray(z, dtype=np.float64)
    return np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def cv_squared_grad(v) -> np.ndarray:
    """Gradient of CV^2(v) = Var(v) / mean(v)^2 (population variance) with
    respect to each v_i: 2 / (n m^2) * (v_i - m - Var / m); zero when the mean
    is zero (where CV^2 is defined as 0)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.size
    if n == 0:
        return np.zeros(0)
    m = v.mean()
    if m == 0.0:
        return np.zeros(n)
    var = ((v - m) ** 2).mean()
    return 2.0 / (n * m * m) * (v - m - var / m)


def rank_experts(H: np.ndarray, k: int):
    """The experts ranked k-th and (k+1)-th by (score descending, index
    ascending), the ones whose scores are the thresholds kth and k1th of
    keep_top_k; -1 where there is no (k+1)-th (k == E)."""
    H = np.asarray(H, dtype=np.float64)
    T, E = H.shape
    order = np.argsort(-H, axis=1, kind="stable")
    jk = order[:, k - 1] if T else np.zeros(0, dtype=np.int64)
    jk1 = order[:, k] if (T and k < E) else np.full(T, -1)
    return jk, jk1


def expert_relu_backward(X, w1_e, w2_e, dY):
    """E(X) = max(X W1^T, 0) W2^T.  Returns dX, dW1 [h][d], dW2 [d][h]."""
    X, w1_e, w2_e, dY = _f64(X), _f64(w1_e), _f64(w2_e), _f64(dY)
    P = X @ w1_e.T
    hid = np.maximum(P, 0.0)
    dhid = dY @ w2_e
    dP = dhid * (P > 0.0)
    return dP @ w1_e, dP.T @ X, dY.T @ hid


def expert_swiglu_backward(X, w1_e, w3_e, w2_e, dY):
    """E(X) = (silu(X W1^T) * (X W3^T)) W2^T.  Returns dX, dW1, dW3, dW2.
    silu'(a) = s (1 + a (1 - s)) with s = sigmoid(a)."""
    X, w1_e, w3_e, w2_e, dY = _f64(X), _f64(w1_e), _f64(w3_e), _f64(w2_e), _f64(dY)
    a = X @ w1_e.T
    b = X @ w3_e.T
    s = sigmoid(a)
    hid = a * s * b
    dhid = dY @ w2_e
    da = dhid * b * s * (1.0 + a * (1.0 - s))
    db = dhid * a * s
    return da @ w1_e + db @ w3_e, da.T @ X, db.T @ X, dY.T @ hid


def backward(inp: Dict, cfg, dy, w_importance=1.0, w_load=1.0) -> Dict:
    """Gradients of L (see above), flat or hierarchical gate, ReLU or SwiGLU
    experts.

    Returns dx [T][d], dw_gate [E][d], dw_noise [E][d] (None without noise),
    dbias [E] (None for the hierarchy, which has no bias), dw1 [E][h][d], dw3
    (SwiGLU, else None), dw2 [E][d][h], for the hierarchy dw_gate_p [G][d] and
    dw_noise_p [G][d], and the intermediates dgate [T][k] (gradient of the
    kept gates) and dH [T][E] (gradient of the noisy scores; the hierarchy
    adds dH_p [T][G]).
    """
    x = _f64(inp["x"])
    dy = _f64(dy)
    fw = forward(inp, cfg, w_importance, w_load)
    g = fw["gate_info"]
    idx, gates, inv = fw["idx"], fw["gates"], fw["inv"]
    T, k = idx.shape

    # combine: y_t = sum over the kept slots of gate[t,s] * y_sorted[inv[t,s]]
    inv2 = inv.reshape(T, k)
    y_rows = np.zeros((T, k, dy.shape[1]))
    kept_slot = inv2 >= 0
    y_rows[kept_slot] = fw["y_sorted"][inv2[kept_slot]]   # dropped slots add nothing
    dgate = np.einsum("tsd,td->ts", y_rows, dy) if T else np.zeros((0, k))
    # importance: d Importance_e / d G[t,e] = 1 for every kept (t, e)
    dgate = dgate + w_importance * cv_squared_grad(fw["importance"])[idx]
    if cfg.n_groups:
        res = _hier_gate_backward(inp, cfg, x, g, dgate)
    else:
        res = _flat_gate_backward(inp, cfg, x, fw, dgate, w_load)
    dx = res.pop("dx")
    _expert_backward(inp, cfg, x, dy, fw, dx, res)
    return dict(dx=dx, dgate=dgate, forward=fw, **res)


def _flat_gate_backward(inp, cfg, x, fw, dgate, w_load):
    """The flat gate's share: softmax over the kept scores, the smooth load,
    the noisy score, the two projections and the bias."""
    g = fw["gate_info"]
    idx, gates = fw["idx"], fw["gates"]
    T, k = idx.shape
    E = cfg.n_experts
    rows = np.arange(T)
    # softmax over the kept scores
    dH_kept = gates * (dgate - (gates * dgate).sum(axis=1, keepdims=True))
    dH = np.zeros((T, E))
    for s in range(k):
        dH[rows, idx[:, s]] += dH_kept[:, s]

    clean, sp, H = g["clean"], g["sp"], g["H"]
    dclean = np.zeros((T, E))
    dsp = np.zeros((T, E))
    if sp is not None:
        # smooth load: Load_e = sum_t Phi(z), z = (clean - theta) / sp, theta the
        # k-th largest score among the other experts, the score of the expert
        # ranked k+1 when e is kept and of the one ranked k otherwise
        kept = np.zeros((T, E), dtype=bool)
        for s in range(k):
            kept[rows, idx[:, s]] = True
        jk, jk1 = rank_experts(H, k)
        theta = np.where(kept, g["k1th"][:, None], g["kth"][:, None])
        with np.errstate(invalid="ignore"):
            z = (clean - theta) / sp
        dload = w_load * cv_squared_grad(fw["load"])
        dz = dload[None, :] * np.where(np.isfinite(z), normal_pdf(np.where(np.isfinite(z), z, 0.0)), 0.0)
        zf = np.where(np.isfinite(z), z, 0.0)
        dclean += dz / sp
        dsp += -dz * zf / sp
        dtheta = -dz / sp
        dH[rows, jk] += np.where(kept, 0.0, dtheta).sum(axis=1)
        has_k1 = jk1 >= 0
        dH[rows[has_k1], jk1[has_k1]] += np.where(kept, dtheta, 0.0).sum(axis=1)[has_k1]
        # H = clean + eps * sp
        dclean += dH
        dsp += dH * _f64(inp["eps"])
        raw = x @ _f64(inp["w_noise"]).T
        draw = dsp * sigmoid(raw)
    else:
        dclean += dH
        draw = None

    # clean = x W_g^T + bias, raw = x W_noise^T
    dw_gate = dclean.T @ x
    dw_noise = draw.T @ x if draw is not None else None
    dbias = dclean.sum(axis=0)
    dx = dclean @ _f64(inp["w_gate"])
    if draw is not None:
        dx = dx + draw @ _f64(inp["w_noise"])
    return dict(dx=dx, dw_gate=dw_gate, dw_noise=dw_noise, dbias=dbias, dH=dH)


def _hier_gate_backward(inp, cfg, x, g, dgate):
    """The hierarchy's share.  A kept gate is gp[a] * gs[a, b]: the primary
    softmax weight of kept group a times the secondary softmax weight of its
    kept expert b, so d gs[a, b] = dgate * gp[a] and d gp[a] = sum over b of
    dgate * gs[a, b]; each level then differentiates like a flat gate over its
    kept scores (softmax, noisy score, projections).  The hierarchy's load is
    a hard count, so no load gradient reaches either level."""
    T, k = g["idx"].shape
    E, G = cfg.n_experts, cfg.n_groups
    Eg, kg, kpg = E // G, cfg.k_groups, cfg.k_per_group
    prim = g["primary"]
    wg, wn = _f64(inp["w_gate"]), _f64(inp.get("w_noise"))
    wgp, wnp = _f64(inp["w_gate_p"]), _f64(inp.get("w_noise_p"))
    eps, eps_p = _f64(inp.get("eps")), _f64(inp.get("eps_p"))
    noisy = wn is not None and eps is not None
    noisy_p = wnp is not None and eps_p is not None
    dclean_p = np.zeros((T, G))
    draw_p = np.zeros((T, G))
    dclean = np.zeros((T, E))
    draw = np.zeros((T, E))
    for t in range(T):
        gp = prim["gates"][t]                       # [kg], kept groups ascending
        dgp = np.zeros(kg)
        for a in range(kg):
            grp = int(prim["idx"][t, a])
            sub = slice(grp * Eg, (grp + 1) * Eg)
            sec = flat_gate(x[t:t + 1], wg[sub], None if not noisy else wn[sub], None,
                            None if not noisy else eps[t:t + 1, grp, :], kpg)
            gs = sec["gates"][0]                    # [kpg], kept experts ascending
            dg = dgate[t, a * kpg:(a + 1) * kpg]
            dgp[a] = (dg * gs).sum()
            dgs = dg * gp[a]
            dHs = gs * (dgs - (gs * dgs).sum())
            for b in range(kpg):
                j = int(sec["idx"][0, b])
                e = grp * Eg + j
                dclean[t, e] += dHs[b]
                if noisy:
                    # H = clean + eps * softplus(raw): d raw = dH * eps * sigmoid(raw)
                    raw = float(x[t] @ wn[e])
                    draw[t, e] += dHs[b] * eps[t, grp, j] * sigmoid(raw)
        dHp = gp * (dgp - (gp * dgp).sum())
        for a in range(kg):
            grp = int(prim["idx"][t, a])
            dclean_p[t, grp] += dHp[a]
            if noisy_p:
                raw = float(x[t] @ wnp[grp])
                draw_p[t, grp] += dHp[a] * eps_p[t, grp] * sigmoid(raw)
    dx = dclean_p @ wgp + dclean @ wg
    res = dict(dw_gate_p=dclean_p.T @ x, dw_gate=dclean.T @ x, dbias=None,
               dH=dclean, dH_p=dclean_p, dw_noise=None, dw_noise_p=None)
    if noisy:
        dx = dx + draw @ wn
        res["dw_noise"] = draw.T @ x
    if noisy_p:
        dx = dx + draw_p @ wnp
        res["dw_noise_p"] = draw_p.T @ x
    res["dx"] = dx
    return res


def _expert_backward(inp, cfg, x, dy, fw, dx, res):
    """The experts' share, added into dx; writes dw1, dw2 (dw3) into res.
    The rows of expert e are the tokens perm[p] // k, and the gradient
    flowing into row p is gate[t,s] * dy[t]."""
    gates = fw["gates"]
    k = gates.shape[1]
    E = cfg.n_experts
    w1, w2 = _f64(inp["w1"]), _f64(inp["w2"])
    w3 = _f64(inp.get("w3"))
    perm, offsets = fw["perm"], fw["offsets"]
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    dw3 = np.zeros_like(w3) if w3 is not None else None
    flat_gates = gates.reshape(-1)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        a = perm[lo:hi]
        toks = a // k
        X = x[toks]
        dY = flat_gates[a][:, None] * dy[toks]
        if w3 is None:
            dX, dw1[e], dw2[e] = expert_relu_backward(X, w1[e], w2[e], dY)
        else:
            dX, dw1[e], dw3[e], dw2[e] = expert_swiglu_backward(X, w1[e], w3[e], w2[e], dY)
        np.add.at(dx, toks, dX)
    res.update(dw1=dw1, dw2=dw2, dw3=dw3)


# ---------------------------------------------------------------------------
# Noise drawn from a counter-based generator  [MoE lesson, section 四: a fresh
# standard-normal draw per call]
#
# Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
# Easy as 1, 2, 3", SC 2011): a 128-bit counter and a 64-bit key; ten rounds,
# each multiplying counter words 0 and 2 by two fixed 32-bit constants and
# mixing the high halves with the other words and the key, the key then
# bumped by two Weyl constants.  Element i of a noise row `row` (group `sub`,
# stream `stream`: 0 flat / secondary, 1 primary) takes the Philox output of
# counter (i // 4, row, sub, stream) under key (seed low, seed high): words
# (0, 1) feed elements 4q, 4q+1 and words (2, 3) elements 4q+2, 4q+3 through
# the Box-Muller transform r = sqrt(-2 ln u_a), n = r cos(2 pi u_b) (even
# element) or r sin(2 pi u_b) (odd), u = (top 23 bits + 1/2) / 2^23, which
# float32 holds exactly.
# ---------------------------------------------------------------------------

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85


def philox4x32_10(ctr, key):
    """ctr: uint [..., 4], key: uint [..., 2] (broadcast) -> uint32 [..., 4]."""
    c = [np.asarray(ctr, dtype=np.uint64)[..., i] & 0xFFFFFFFF for i in range(4)]
    key = np.asarray(key, dtype=np.uint64)
    k0, k1 = key[..., 0] & 0xFFFFFFFF, key[..., 1] & 0xFFFFFFFF
    mask = np.uint64(0xFFFFFFFF)
    for _ in range(10):
        p0 = np.uint64(PHILOX_M0) * c[0]
        p1 = np.uint64(PHILOX_M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c = [(hi1 ^ c[1] ^ k0) & mask, lo1, (hi0 ^ c[3] ^ k1) & mask, lo0]
        k0 = (k0 + np.uint64(PHILOX_W0)) & mask
        k1 = (k1 + np.uint64(PHILOX_W1)) & mask
    return np.stack(c, axis=-1).astype(np.uint32)


def uniform23(x):
    """(top 23 bits of x + 1/2) / 2^23: in (0, 1), exact in float32."""
    return ((np.asarray(x, dtype=np.uint32) >> np.uint32(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def philox_normals(rows, n, seed, sub=0, stream=0):
    """Standard normals [len(rows)][n] of the given noise rows (see above)."""
    rows = np.asarray(rows, dtype=np.uint64)
    i = np.arange(n, dtype=np.uint64)
    q = i >> np.uint64(2)
    ctr = np.zeros((rows.size, n, 4), dtype=np.uint64)
    ctr[..., 0] = q[None, :]
    ctr[..., 1] = rows[:, None]
    ctr[..., 2] = np.uint64(sub)
    ctr[..., 3] = np.uint64(stream)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    out = philox4x32_10(ctr, key)
    j = (i & np.uint64(3)).astype(np.int64)
    pair = j >> 1
    xa = np.where(pair == 0, out[..., 0], out[..., 2])
    xb = np.where(pair == 0, out[..., 1], out[..., 3])
    r = np.sqrt(-2.0 * np.log(uniform23(xa)))
    ang = 2.0 * math.pi * uniform23(xb)
    return np.where((j & 1) == 0, r * np.cos(ang), r * np.sin(ang))


def draw_noise(cfg, seed) -> Dict:
    """The noise tensors of one layer call drawn from `seed`: eps [T][E]
    (flat), or eps_p [T][G] and eps [T][G][Eg] (hierarchy)."""
    T = cfg.tokens
    rows = np.arange(T)
    if not cfg.n_groups:
        return dict(eps=philox_normals(rows, cfg.n_experts, seed, 0, 0), eps_p=None)
    G, Eg = cfg.n_groups, cfg.n_experts // cfg.n_groups
    eps = np.stack([philox_normals(rows, Eg, seed, g, 0) for g in range(G)], axis=1)
    return dict(eps=eps, eps_p=philox_normals(rows, G, seed, 0, 1))
