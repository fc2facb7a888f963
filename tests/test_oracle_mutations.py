"""Evidence that the oracle's pins have teeth: each case plants one plausible
mistake in the oracle (a dropped term, a flipped sign, a wrong index or
tie-break, a transposed operand, an off-by-one rank, a different variance) and
checks that the pins named beside it fail on the planted oracle.  The mistakes
live in this file only; the oracle itself is patched for the duration of one
test and restored by pytest.  CPU only."""
import importlib.util
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import oracle.moe_oracle as om

_HERE = os.path.dirname(os.path.abspath(__file__))


def _load(name):
    spec = importlib.util.spec_from_file_location("_" + name, os.path.join(_HERE, name + ".py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


pins = _load("test_oracle_pins")
bpins = _load("test_oracle_backward_pins")
cpins = _load("test_oracle_capacity_pins")
npins = _load("test_oracle_noise_pins")
mpins = _load("test_oracle_mask_pins")

_orig = {name: getattr(om, name) for name in dir(om) if not name.startswith("__")}


def _cases(fn):
    """Argument tuples of a pin: one per parametrize value, else one empty."""
    for mark in getattr(fn, "pytestmark", []):
        if mark.name == "parametrize":
            return [(v,) for v in mark.args[1]]
    return [()]


def _pin_fails(name):
    fn = (getattr(pins, name, None) or getattr(bpins, name, None) or getattr(cpins, name, None)
          or getattr(npins, name, None) or getattr(mpins, name))
    for args in _cases(fn):
        try:
            fn(*args)
        except Exception:  # an assertion or a crash: either way the pin rejects it
            return True
    return False


def _top_k_from_order(H, order, k):
    """The remainder of KeepTopK once a descending order is chosen."""
    T, E = H.shape
    idx = np.sort(order[:, :k], axis=1).astype(np.int32)
    rows = np.arange(T)
    kth = H[rows, order[:, k - 1]] if T else np.zeros(0)
    k1th = H[rows, order[:, k]] if (T and k < E) else np.full(T, -np.inf)
    with np.errstate(invalid="ignore"):
        return idx, kth, k1th, kth - k1th


# ------------------------------------------------------------ mistakes ----

def noise_term_dropped(x, w_gate, w_noise=None, bias=None, eps=None):
    clean, sp, _ = _orig["noisy_logits"](x, w_gate, w_noise, bias, eps)
    return clean, sp, clean.copy()


def bias_dropped(x, w_gate, w_noise=None, bias=None, eps=None):
    return _orig["noisy_logits"](x, w_gate, w_noise, None, eps)


def noise_scale_from_clean_table(x, w_gate, w_noise=None, bias=None, eps=None):
    return _orig["noisy_logits"](x, w_gate, w_gate if w_noise is not None else None, bias, eps)


def softplus_sign_flipped(z):
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(-z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def softplus_linear_part_dropped(z):
    z = np.asarray(z, dtype=np.float64)
    return np.log1p(np.exp(-np.abs(z)))


def cdf_argument_sign_flipped(z):
    return 0.5 * scipy.special.erfc(np.asarray(z, dtype=np.float64) / math.sqrt(2.0))


def cdf_without_root_two(z):
    return 0.5 * scipy.special.erfc(-np.asarray(z, dtype=np.float64))


def silu_with_negated_sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return z * (0.5 * (1.0 - np.tanh(0.5 * z)))


def ties_to_higher_index(H, k):
    H = np.asarray(H, dtype=np.float64)
    E = H.shape[1]
    order = E - 1 - np.argsort(-H[:, ::-1], axis=1, kind="stable")
    return _top_k_from_order(H, order, k)


def kth_and_k1th_swapped(H, k):
    idx, kth, k1th, margin = _orig["keep_top_k"](H, k)
    return idx, k1th, kth, margin


def kept_in_score_order(H, k):
    H = np.asarray(H, dtype=np.float64)
    order = np.argsort(-H, axis=1, kind="stable")
    idx, kth, k1th, margin = _top_k_from_order(H, order, k)
    return order[:, :k].astype(np.int32), kth, k1th, margin


def softmax_over_all_experts(H, idx):
    H = np.asarray(H, dtype=np.float64)
    if H.shape[0] == 0:
        return np.zeros(idx.shape)
    P = scipy.special.softmax(H, axis=1)
    return np.take_along_axis(P, idx.astype(np.int64), axis=1)


def route_capacity_keeps_latest(idx, n_experts, capacity=0):
    """Keeps the last `capacity` tokens of an expert instead of the first."""
    if capacity <= 0:
        return _orig["route"](idx, n_experts)
    T, k = idx.shape
    flipped = idx[::-1]
    counts, offsets, perm_f, inv_f = _orig["route"](flipped, n_experts, capacity)
    inv = np.full(T * k, -1, dtype=np.int32)
    perm = np.zeros_like(perm_f)
    for a_f in range(T * k):
        t_f, s_ = divmod(a_f, k)
        if inv_f[a_f] >= 0:
            a = (T - 1 - t_f) * k + s_
            inv[a] = inv_f[a_f]
            perm[inv_f[a_f]] = a
    return counts, offsets, perm, inv


def route_capacity_off_by_one(idx, n_experts, capacity=0):
    return _orig["route"](idx, n_experts, capacity + 1 if capacity > 0 else 0)


def combine_dropped_slot_reads_last_row(y_sorted, inv, gates):
    """A dropped slot (-1) indexes the last routed row instead of adding nothing."""
    gates = np.asarray(gates, dtype=np.float64)
    T, k = gates.shape
    y = np.zeros((T, y_sorted.shape[1]))
    inv2 = np.asarray(inv).reshape(T, k)
    for s_ in range(k):
        y += gates[:, s_:s_ + 1] * y_sorted[inv2[:, s_]]
    return y


def philox_without_key_bump(ctr, key):
    """Ten rounds that reuse the first round key."""
    c = [np.asarray(ctr, dtype=np.uint64)[..., i] for i in range(4)]
    key = np.asarray(key, dtype=np.uint64)
    k0, k1 = key[..., 0], key[..., 1]
    mask = np.uint64(0xFFFFFFFF)
    for _ in range(10):
        p0 = np.uint64(om.PHILOX_M0) * c[0]
        p1 = np.uint64(om.PHILOX_M1) * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & mask, p1 & mask,
             ((p0 >> np.uint64(32)) ^ c[3] ^ k1) & mask, p0 & mask]
    return np.stack(c, axis=-1).astype(np.uint32)


def philox_words_of_product_swapped(ctr, key):
    out = _orig["philox4x32_10"](ctr, key)
    return out[..., [1, 0, 3, 2]]


def uniform_from_24_bits(x):
    return ((np.asarray(x, dtype=np.uint32) >> np.uint32(8)).astype(np.float64) + 0.5) * 2.0 ** -24


def normals_sin_and_cos_swapped(rows, n, seed, sub=0, stream=0):
    z = _orig["philox_normals"](rows, n, seed, sub, stream)
    m = n - n % 2
    out = z.copy()
    out[:, 0:m:2], out[:, 1:m:2] = z[:, 1:m:2], z[:, 0:m:2]
    return out


def route_tokens_descending(idx, n_experts):
    T, k = idx.shape
    counts, offsets, _, _ = _orig["route"](idx, n_experts)
    fill = offsets[:-1].astype(np.int64).copy()
    perm = np.zeros(T * k, dtype=np.int32)
    inv = np.zeros(T * k, dtype=np.int32)
    for t in reversed(range(T)):
        for s in range(k):
            p = fill[idx[t, s]]
            fill[idx[t, s]] += 1
            perm[p] = t * k + s
            inv[t * k + s] = p
    return counts, offsets, perm, inv


def route_inclusive_offsets(idx, n_experts):
    counts, offsets, perm, inv = _orig["route"](idx, n_experts)
    return counts, np.append(offsets[1:], offsets[-1]).astype(np.int32), perm, inv


def expert_without_relu(X, w1_e, w2_e):
    X = om._f64(X)
    return (X @ om._f64(w1_e).T) @ om._f64(w2_e).T


def swiglu_gate_and_up_swapped(X, w1_e, w3_e, w2_e):
    return _orig["expert_swiglu"](X, w3_e, w1_e, w2_e)


def experts_fed_assignment_index(x, perm, offsets, k, w1, w2, w3=None):
    """Rows gathered by assignment number t*k+s instead of token t."""
    x = om._f64(x)
    E = len(offsets) - 1
    y = np.zeros((int(offsets[-1]), om._f64(w2[0]).shape[0]))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi] = om.expert_apply(x[np.asarray(perm[lo:hi]) % x.shape[0]], e, w1, w2, w3)
    return y


def combine_without_gates(y_sorted, inv, gates):
    return _orig["combine"](y_sorted, inv, np.ones_like(np.asarray(gates, dtype=np.float64)))


def combine_through_perm(y_sorted, inv, gates):
    perm = np.argsort(np.asarray(inv))   # the inverse of inv, used where inv belongs
    return _orig["combine"](y_sorted, perm, gates)


def cv2_sample_variance(v):
    v = np.asarray(v, dtype=np.float64)
    if v.size < 2 or v.mean() == 0.0:
        return 0.0
    return float(v.var(ddof=1) / v.mean() ** 2)


def cv2_not_squared_mean(v):
    v = np.asarray(v, dtype=np.float64)
    if v.size == 0 or v.mean() == 0.0:
        return 0.0
    return float(v.var() / abs(v.mean()))


def importance_counts_rows(idx, gates, n_experts):
    return _orig["importance"](idx, np.ones_like(gates), n_experts)


def load_theta_swapped(clean, sp, H, idx, kth, k1th):
    return _orig["load_estimate"](clean, sp, H, idx, k1th, kth)


def load_without_noise_scale(clean, sp, H, idx, kth, k1th):
    return _orig["load_estimate"](clean, np.ones_like(sp), H, idx, kth, k1th)


def loss_weights_swapped(n_experts, idx, gates, counts, gate_info=None,
                         w_importance=1.0, w_load=1.0):
    return _orig["balance_stats"](n_experts, idx, gates, counts, gate_info, w_load, w_importance)


def hier_primary_gate_only(x, w_gate_p, w_noise_p, eps_p, w_gate, w_noise, eps,
                           n_groups, k_groups, k_per_group):
    h = _orig["hier_gate"](x, w_gate_p, w_noise_p, eps_p, w_gate, w_noise, eps,
                           n_groups, k_groups, k_per_group)
    h["gates"] = np.repeat(h["primary"]["gates"], k_per_group, axis=1)
    return h


def hier_expert_index_transposed(x, w_gate_p, w_noise_p, eps_p, w_gate, w_noise, eps,
                                 n_groups, k_groups, k_per_group):
    """Global expert j*n_groups + g instead of g*Eg + j."""
    h = _orig["hier_gate"](x, w_gate_p, w_noise_p, eps_p, w_gate, w_noise, eps,
                           n_groups, k_groups, k_per_group)
    Eg = om._f64(w_gate).shape[0] // n_groups
    g, j = h["idx"] // Eg, h["idx"] % Eg
    h["idx"] = (j * n_groups + g).astype(np.int32)
    return h


def cv2_grad_without_mean_term(v):
    v = np.asarray(v, dtype=np.float64)
    if v.size == 0 or v.mean() == 0.0:
        return np.zeros(v.size)
    m = v.mean()
    return 2.0 / (v.size * m * m) * (v - m)


def pdf_without_normalisation(z):
    z = np.asarray(z, dtype=np.float64)
    return np.exp(-0.5 * z * z)


def rank_k_and_k1_swapped(H, k):
    jk, jk1 = _orig["rank_experts"](H, k)
    return np.where(jk1 >= 0, jk1, jk), np.where(jk1 >= 0, jk, -1)


def relu_backward_weights_from_pre_activation(X, w1_e, w2_e, dY):
    dX, dW1, _ = _orig["expert_relu_backward"](X, w1_e, w2_e, dY)
    X, w1_e, dY = om._f64(X), om._f64(w1_e), om._f64(dY)
    return dX, dW1, dY.T @ (X @ w1_e.T)


def relu_backward_without_mask(X, w1_e, w2_e, dY):
    X, w1_e, w2_e, dY = om._f64(X), om._f64(w1_e), om._f64(w2_e), om._f64(dY)
    dP = dY @ w2_e
    return dP @ w1_e, dP.T @ X, dY.T @ np.maximum(X @ w1_e.T, 0.0)


def swiglu_backward_sigmoid_as_silu_derivative(X, w1_e, w3_e, w2_e, dY):
    X, w1_e, w3_e, w2_e, dY = (om._f64(a) for a in (X, w1_e, w3_e, w2_e, dY))
    a, b = X @ w1_e.T, X @ w3_e.T
    s = om.sigmoid(a)
    dhid = dY @ w2_e
    da, db = dhid * b * s, dhid * a * s
    return da @ w1_e + db @ w3_e, da.T @ X, db.T @ X, dY.T @ (a * s * b)


def noise_scale_slope_one(z):
    return np.ones_like(np.asarray(z, dtype=np.float64))


def hier_backward_noise_of_next_group(inp, cfg, x, g, dgate):
    """The secondary noise read from a neighbouring group's slice."""
    eps = inp.get("eps")
    inp = dict(inp, eps=None if eps is None else np.roll(om._f64(eps), 1, axis=1))
    return _orig["_hier_gate_backward"](inp, cfg, x, g, dgate)


def hier_backward_primary_level_dropped(inp, cfg, x, g, dgate):
    """No gradient for the primary (group) tables."""
    res = _orig["_hier_gate_backward"](inp, cfg, x, g, dgate)
    res["dw_gate_p"] = np.zeros_like(res["dw_gate_p"])
    if res["dw_noise_p"] is not None:
        res["dw_noise_p"] = np.zeros_like(res["dw_noise_p"])
    return res


def noise_primary_on_stream_zero(cfg, seed):
    """The primary noise drawn on the secondary stream (counter word 3 = 0)."""
    d = _orig["draw_noise"](cfg, seed)
    if cfg.n_groups:
        d["eps_p"] = om.philox_normals(np.arange(cfg.tokens), cfg.n_groups, seed, 0, 0)
    return d


def noise_flat_rows_from_one(cfg, seed):
    """Token t's flat noise row read at counter row t + 1."""
    d = _orig["draw_noise"](cfg, seed)
    if not cfg.n_groups:
        d["eps"] = om.philox_normals(np.arange(1, cfg.tokens + 1), cfg.n_experts, seed, 0, 0)
    return d


def noise_group_in_stream_word(cfg, seed):
    """The secondary noise of group g with g in the stream word, not the group word."""
    d = _orig["draw_noise"](cfg, seed)
    if cfg.n_groups:
        Eg = cfg.n_experts // cfg.n_groups
        rows = np.arange(cfg.tokens)
        d["eps"] = np.stack([om.philox_normals(rows, Eg, seed, 0, g) for g in
                             range(cfg.n_groups)], axis=1)
    return d


def batch_mask_ties_to_higher_token(H, m):
    H = np.asarray(H, dtype=np.float64)
    T, E = H.shape
    keep = np.zeros((T, E), dtype=bool)
    for e in range(E):
        order = (T - 1 - np.argsort(-H[::-1, e], kind="stable"))
        keep[order[:min(m, T)], e] = True
    return keep


def batch_mask_keeps_one_more(H, m):
    return _orig["batch_mask"](H, m + 1)


def threshold_strictly_above(H, theta):
    return np.asarray(H, dtype=np.float64) > np.asarray(theta, dtype=np.float64)[None, :]


def masked_softmax_over_all_experts(H, keep):
    H = np.asarray(H, dtype=np.float64)
    w = np.exp(H - H.max(axis=1, keepdims=True))
    return np.where(keep, w / w.sum(axis=1, keepdims=True), 0.0)


def masked_route_tokens_descending(keep, capacity=0):
    T = keep.shape[0]
    counts, offsets, perm, pos = _orig["masked_route"](keep[::-1], capacity)
    perm = (T - 1 - perm).astype(np.int32)
    return counts, offsets, perm, pos[::-1]


def masked_route_capacity_keeps_latest(keep, capacity=0):
    if capacity <= 0:
        return _orig["masked_route"](keep, capacity)
    keep = keep.copy()
    for e in range(keep.shape[1]):
        toks = np.nonzero(keep[:, e])[0]
        keep[toks[:max(0, toks.size - capacity)], e] = False
    return _orig["masked_route"](keep, 0)


# (function patched, mistake, pins that must reject it)
MUTATIONS = [
    ("noisy_logits", noise_term_dropped, ["test_noisy_logits_hand_example"]),
    ("noisy_logits", bias_dropped, ["test_noisy_logits_hand_example"]),
    ("noisy_logits", noise_scale_from_clean_table, ["test_noisy_logits_hand_example"]),
    ("softplus", softplus_sign_flipped, ["test_softplus_closed_forms", "test_noisy_logits_hand_example"]),
    ("softplus", softplus_linear_part_dropped, ["test_softplus_closed_forms", "test_noisy_logits_hand_example"]),
    ("normal_cdf", cdf_argument_sign_flipped, ["test_normal_cdf_closed_forms", "test_load_estimate_monte_carlo"]),
    ("normal_cdf", cdf_without_root_two, ["test_normal_cdf_closed_forms", "test_load_two_experts_top1_closed_form"]),
    ("silu", silu_with_negated_sigmoid, ["test_silu_closed_forms", "test_single_expert_swiglu_matches_torch"]),
    ("keep_top_k", ties_to_higher_index, ["test_ties_prefer_lower_index",
                                          "test_zero_tables_give_uniform_gates_and_lowest_index_ties"]),
    ("keep_top_k", kth_and_k1th_swapped, ["test_top_k_equals_brute_force_best_subset",
                                          "test_load_estimate_monte_carlo"]),
    ("keep_top_k", kept_in_score_order, ["test_top_k_equals_brute_force_best_subset",
                                         "test_gate_invariants_random"]),
    ("kept_softmax", softmax_over_all_experts, ["test_worked_example_from_the_lesson_page",
                                                "test_gate_invariants_random"]),
    ("route", route_tokens_descending, ["test_route_hand_example", "test_route_invariants_random"]),
    ("route", route_inclusive_offsets, ["test_route_hand_example", "test_route_invariants_random"]),
    ("expert_relu", expert_without_relu, ["test_single_expert_is_a_plain_relu_ffn",
                                          "test_dense_mixture_when_k_equals_E"]),
    ("expert_swiglu", swiglu_gate_and_up_swapped, ["test_single_expert_swiglu_matches_torch"]),
    ("run_experts", experts_fed_assignment_index, ["test_sparse_layer_equals_dense_brute_force",
                                                   "test_dense_mixture_when_k_equals_E"]),
    ("combine", combine_without_gates, ["test_combine_hand_example",
                                        "test_sparse_layer_equals_dense_brute_force"]),
    ("combine", combine_through_perm, ["test_combine_hand_example",
                                       "test_sparse_layer_equals_dense_brute_force"]),
    ("cv_squared", cv2_sample_variance, ["test_cv_squared_closed_forms"]),
    ("cv_squared", cv2_not_squared_mean, ["test_cv_squared_closed_forms"]),
    ("importance", importance_counts_rows, ["test_importance_sums_to_token_count"]),
    ("load_estimate", load_theta_swapped, ["test_load_two_experts_top1_closed_form",
                                           "test_load_estimate_monte_carlo"]),
    ("load_estimate", load_without_noise_scale, ["test_load_two_experts_top1_closed_form"]),
    ("balance_stats", loss_weights_swapped, ["test_balance_loss_weights"]),
    ("hier_gate", hier_primary_gate_only, ["test_hierarchy_constructed_case",
                                           "test_hierarchy_invariants_random"]),
    ("hier_gate", hier_expert_index_transposed, ["test_hierarchy_constructed_case",
                                                 "test_hierarchy_invariants_random"]),
    # capacity
    ("route", route_capacity_keeps_latest, ["test_route_capacity_hand_example",
                                            "test_capacity_invariants_random",
                                            "test_capacity_layer_equals_brute_force"]),
    ("route", route_capacity_off_by_one, ["test_route_capacity_hand_example",
                                          "test_capacity_invariants_random"]),
    ("combine", combine_dropped_slot_reads_last_row, ["test_capacity_layer_equals_brute_force"]),
    # counter-based noise
    ("philox4x32_10", philox_without_key_bump, ["test_philox_known_answers"]),
    ("philox4x32_10", philox_words_of_product_swapped, ["test_philox_known_answers"]),
    ("uniform23", uniform_from_24_bits, ["test_uniform23_range_and_exactness"]),
    ("philox_normals", normals_sin_and_cos_swapped, ["test_normals_follow_the_counter_layout"]),
    ("draw_noise", noise_primary_on_stream_zero, ["test_draw_noise_counter_layout"]),
    ("draw_noise", noise_flat_rows_from_one, ["test_draw_noise_counter_layout"]),
    ("draw_noise", noise_group_in_stream_word, ["test_draw_noise_counter_layout"]),
    ("batch_mask", batch_mask_ties_to_higher_token, ["test_batch_mask_hand_example",
                                                     "test_every_expert_keeps_exactly_m_of_its_best"]),
    ("batch_mask", batch_mask_keeps_one_more, ["test_batch_mask_hand_example",
                                               "test_every_expert_keeps_exactly_m_of_its_best",
                                               "test_calibrated_thresholds_reproduce_the_batch_mask"]),
    ("threshold_mask", threshold_strictly_above, ["test_threshold_mask_hand_example",
                                                  "test_calibrated_thresholds_reproduce_the_batch_mask"]),
    ("masked_gates", masked_softmax_over_all_experts, ["test_batch_mask_hand_example",
                                                       "test_masked_gates_invariants"]),
    ("masked_route", masked_route_tokens_descending, ["test_batch_mask_hand_example"]),
    ("masked_route", masked_route_capacity_keeps_latest, ["test_batch_mask_hand_example",
                                                          "test_masked_layer_equals_dense_mixture_over_kept_pairs"]),
    # backward
    ("cv_squared_grad", cv2_grad_without_mean_term, ["test_cv_squared_gradient_closed_forms",
                                                     "test_gradients_match_central_differences"]),
    ("normal_pdf", pdf_without_normalisation, ["test_normal_pdf_and_sigmoid_closed_forms",
                                               "test_gradients_match_central_differences"]),
    ("rank_experts", rank_k_and_k1_swapped, ["test_rank_experts_follow_the_tie_break",
                                             "test_gradients_match_central_differences"]),
    ("expert_relu_backward", relu_backward_weights_from_pre_activation,
     ["test_single_expert_backward_matches_torch_autograd",
      "test_expert_backward_matches_torch_on_random_rows",
      "test_gradients_match_central_differences"]),
    ("expert_relu_backward", relu_backward_without_mask,
     ["test_single_expert_backward_matches_torch_autograd",
      "test_dense_mixture_backward_matches_torch_autograd"]),
    ("expert_swiglu_backward", swiglu_backward_sigmoid_as_silu_derivative,
     ["test_single_expert_backward_matches_torch_autograd",
      "test_expert_backward_matches_torch_on_random_rows",
      "test_gradients_match_central_differences"]),
    ("sigmoid", noise_scale_slope_one, ["test_normal_pdf_and_sigmoid_closed_forms",
                                        "test_gradients_match_central_differences"]),
    ("_hier_gate_backward", hier_backward_noise_of_next_group,
     ["test_hier_gradients_match_central_differences"]),
    ("_hier_gate_backward", hier_backward_primary_level_dropped,
     ["test_hier_gradients_match_central_differences"]),
]


@pytest.mark.parametrize("target,mistake,catchers", MUTATIONS,
                         ids=[m[1].__name__ for m in MUTATIONS])
def test_pins_reject_planted_mistake(monkeypatch, target, mistake, catchers):
    for name in catchers:
        assert not _pin_fails(name), f"{name} fails on the unplanted oracle"
    monkeypatch.setattr(om, target, mistake)
    monkeypatch.setattr(oracle, target, mistake, raising=False)
    missed = [name for name in catchers if not _pin_fails(name)]
    assert not missed, f"planted {mistake.__name__} in {target} passes {missed}"
