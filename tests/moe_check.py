"""Comparison helpers between the HIP path and the oracle.

Parity bar:
  * routing (kept experts, counts, offsets, perm, inv): bit-exact on every
    token whose k-th vs (k+1)-th noisy score margin (oracle, fp64) is at least
    1e-4; tokens below that margin are excluded and counted;
  * gates: |g - g_ref| <= 1e-5 |g_ref|;
  * layer outputs: |y - y_ref| <= rtol |y_ref| + rtol rms(y_ref), rtol 2e-2
    for bf16 and 1e-4 for fp32;
  * balance statistics: see check_balance.
"""
import numpy as np
import torch

MARGIN = 1e-4
GATE_RTOL = 1e-5


def np_(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").float().numpy() if t.dtype in (torch.bfloat16, torch.float16) \
            else t.detach().to("cpu").numpy()
    return np.asarray(t)


def excluded(ref) -> np.ndarray:
    return np.asarray(ref["margin"]) < MARGIN


def check_gate(idx, gate, ref, excl, thr=None, report=None):
    idx, gate = np_(idx), np_(gate).astype(np.float64)
    inc = ~excl
    bad = np.nonzero((idx[inc] != ref["idx"][inc]).any(axis=1))[0]
    assert bad.size == 0, f"kept experts differ on {bad.size} included tokens, e.g. {np.nonzero(inc)[0][bad[:5]]}"
    g_ref = np.asarray(ref["gates"])[inc]
    err = np.abs(gate[inc] - g_ref)
    assert (err <= GATE_RTOL * np.abs(g_ref)).all(), f"gate rel err {np.max(err / np.abs(g_ref)):.3e}"
    if thr is not None:
        thr = np_(thr).astype(np.float64)
        gi = ref.get("gate_info", ref)
        kth, k1th = np.asarray(gi["kth"])[inc], np.asarray(gi["k1th"])[inc]
        assert np.allclose(thr[inc, 0], kth, rtol=1e-5, atol=1e-5)
        fin = np.isfinite(k1th)
        assert np.allclose(thr[inc, 1][fin], k1th[fin], rtol=1e-5, atol=1e-5)
        assert np.isneginf(thr[inc, 1][~fin]).all()
    if report is not None:
        report["excluded"] = int(excl.sum())
        report["idx_equal_all"] = bool((idx == ref["idx"]).all())
    return True


def check_routing(counts, offsets, perm, inv, idx_gpu, ref, excl, k):
    counts, offsets, perm, inv = np_(counts), np_(offsets), np_(perm), np_(inv)
    idx_gpu = np_(idx_gpu)
    A = perm.size
    # structural invariants of the GPU result itself
    assert offsets[0] == 0 and offsets[-1] == A
    assert (np.diff(offsets) == counts).all()
    assert (np.sort(perm) == np.arange(A)).all()
    assert (perm[inv] == np.arange(A)).all()
    if not excl.any():
        assert (counts == ref["counts"]).all()
        assert (offsets == ref["offsets"]).all()
        assert (perm == ref["perm"]).all()
        assert (inv == ref["inv"]).all()
        return
    # some near-ties: compare what does not depend on them
    inc_asg = np.repeat(~excl, k)
    E = counts.size
    c_inc = np.bincount(idx_gpu.reshape(-1)[inc_asg], minlength=E)
    r_inc = np.bincount(np.asarray(ref["idx"]).reshape(-1)[inc_asg], minlength=E)
    assert (c_inc == r_inc).all()
    keep_g = inc_asg[perm]
    keep_r = inc_asg[np.asarray(ref["perm"])]
    assert (perm[keep_g] == np.asarray(ref["perm"])[keep_r]).all()
    # the GPU grouping of its own selection is exactly the stable one
    _, _, perm_self, _ = _stable_route(idx_gpu, E)
    assert (perm == perm_self).all()


def _stable_route(idx, E):
    import oracle
    return oracle.route(idx.astype(np.int32), E)


def check_close(y, y_ref, rtol, rows=None, what="y"):
    y = np_(y).astype(np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if rows is not None:
        y, y_ref = y[rows], y_ref[rows]
    if y_ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = np.abs(y - y_ref)
    lim = rtol * np.abs(y_ref) + rtol * rms
    worst = float(np.max(err / (np.abs(y_ref) + rms)))
    assert (err <= lim).all(), f"{what}: {int((err > lim).sum())} elements out of tolerance, worst {worst:.3e}"
    return worst


def check_balance(imp, load, out, ref, excl, idx_ref, k1_sets=None, smooth=True, w=(1.0, 1.0)):
    """importance within 1e-5 rel (+ one full gate of slack per excluded token
    on the experts it could swap), load within 1e-5 rel (+ 1e-4 per excluded
    token), the CV^2 values within 1e-4 rel."""
    imp, load, out = np_(imp).astype(np.float64), np_(load).astype(np.float64), np_(out)
    E = imp.size
    slack = np.zeros(E)
    if excl.any() and k1_sets is not None:
        for t in np.nonzero(excl)[0]:
            slack[k1_sets[t]] += 1.0
    imp_ref = np.asarray(ref["importance"])
    assert (np.abs(imp - imp_ref) <= 1e-5 * np.abs(imp_ref) + 1e-5 + slack).all(), \
        f"importance max err {np.max(np.abs(imp - imp_ref)):.3e}"
    load_ref = np.asarray(ref["load"])
    if smooth:
        tol = 1e-5 * np.abs(load_ref) + 1e-5 + 1e-4 * excl.sum()
    else:
        tol = slack
    assert (np.abs(load - load_ref) <= tol).all(), f"load max err {np.max(np.abs(load - load_ref)):.3e}"
    if not excl.any():
        assert out[0] == np.float32(out[0])
        assert abs(out[0] - ref["cv2_importance"]) <= 1e-4 * abs(ref["cv2_importance"]) + 1e-7
        assert abs(out[1] - ref["cv2_load"]) <= 1e-4 * abs(ref["cv2_load"]) + 1e-7
        assert abs(out[2] - (w[0] * ref["cv2_importance"] + w[1] * ref["cv2_load"])) <= \
            1e-4 * abs(out[2]) + 1e-7


def sampled_outputs(cfg, inp, x_cpu, ref, sample):
    """y of the sampled tokens from the oracle's experts, one expert at a
    time over the tokens of the sample that keep it (dropped slots of a
    capacity add nothing): for layers too large for the whole oracle."""
    import oracle
    y_ref = np.zeros((sample.size, cfg.d_model))
    ridx, rg = ref["idx"][sample], ref["gates"][sample]
    kept = np.asarray(ref["inv"]).reshape(-1, cfg.top_k)[sample] >= 0
    for e in np.unique(ridx):
        rows, slots = np.nonzero((ridx == e) & kept)
        if rows.size == 0:
            continue
        w1 = inp["w1"][e].cpu()
        w2 = inp["w2"][e].cpu()
        w3 = inp["w3"][e].cpu() if inp.get("w3") is not None else None
        xe = x_cpu[sample[rows]]
        ye = oracle.expert_swiglu(xe, w1, w3, w2) if w3 is not None else oracle.expert_relu(xe, w1, w2)
        y_ref[rows] += rg[rows, slots][:, None] * ye
    return y_ref


def top_k1_sets(ref, cfg):
    """Per token, the experts an excluded (near-tied) token could swap in:
    its top-(k+1) experts, or every expert of its top-(k_groups+1) groups."""
    g = ref["gate_info"]
    if cfg.hierarchical:
        prim = g["primary"]
        order = np.argsort(-prim["H"], axis=1, kind="stable")[:, :cfg.k_groups + 1]
        Eg = cfg.experts_per_group
        return [np.concatenate([np.arange(q * Eg, (q + 1) * Eg) for q in row]) for row in order]
    order = np.argsort(-g["H"], axis=1, kind="stable")[:, :cfg.top_k + 1]
    return [row for row in order]
