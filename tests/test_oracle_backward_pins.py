"""Pins of the oracle's backward pass against facts fixed outside it: central
finite differences of the oracle's own forward objective (whose forward is
pinned separately), torch's autograd on plain CPU float64 restatements of
special cases (one expert; the dense softmax mixture), closed forms of the
CV^2 gradient, and invariants of the softmax.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from sparsely_gated_mixture_noisy_amd.inputs import MoEConfig, make_inputs, make_upstream


def _cfg(**kw):
    base = dict(name="bw", tokens=6, d_model=5, n_experts=5, d_hidden=7, top_k=2,
                noisy=True, dtype="f32", gate_std=0.6)
    base.update(kw)
    return MoEConfig(**base)


def _np_inputs(cfg, seed):
    inp = make_inputs(cfg, seed=seed)
    out = {}
    for key, v in inp.items():
        out[key] = None if v is None else v.double().numpy().copy()
    rng = np.random.default_rng(seed)
    out["bias"] = (rng.normal(0.0, 0.5, cfg.n_experts) if cfg.bias == "rand"
                   else np.zeros(cfg.n_experts))
    return out


def _objective(inp, cfg, dy, wi, wl):
    fw = oracle.forward(inp, cfg, wi, wl)
    return float((fw["y"] * dy).sum()) + wi * fw["cv2_importance"] + wl * fw["cv2_load"]


def _min_margin(inp, cfg):
    return float(oracle.gate(inp, cfg)["margin"].min())


FD_CASES = [
    dict(ffn="relu", noisy=True, wi=0.7, wl=1.3),
    dict(ffn="swiglu", noisy=True, wi=0.4, wl=0.9),
    dict(ffn="relu", noisy=False, wi=1.1, wl=0.0),
    dict(ffn="relu", noisy=True, wi=0.0, wl=2.0, bias="rand"),
    dict(ffn="swiglu", noisy=True, wi=0.5, wl=0.5, top_k=3),
]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: "-".join(f"{k}={v}" for k, v in c.items()))
def test_gradients_match_central_differences(case):
    """Every gradient the oracle returns equals the central difference of the
    forward objective, element by element, on a tiny layer whose kept sets
    and rank-k experts stay put under the perturbation."""
    case = dict(case)
    wi, wl = case.pop("wi"), case.pop("wl")
    cfg = _cfg(**case)
    for seed in range(50):
        inp = _np_inputs(cfg, seed)
        if _min_margin(inp, cfg) > 5e-3:
            break
    else:
        pytest.fail("no seed with well-separated scores")
    dy = make_upstream(cfg, seed=seed).double().numpy()
    bw = oracle.backward(inp, cfg, dy, wi, wl)
    h = 1e-6
    names = [("x", "dx"), ("w_gate", "dw_gate"), ("bias", "dbias"), ("w1", "dw1"), ("w2", "dw2")]
    if cfg.noisy:
        names.append(("w_noise", "dw_noise"))
    if cfg.ffn == "swiglu":
        names.append(("w3", "dw3"))
    for key, gkey in names:
        base = inp[key]
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            old = base[i]
            base[i] = old + h
            fp = _objective(inp, cfg, dy, wi, wl)
            base[i] = old - h
            fm = _objective(inp, cfg, dy, wi, wl)
            base[i] = old
            num[i] = (fp - fm) / (2 * h)
        ana = bw[gkey]
        scale = max(1.0, np.abs(num).max())
        assert np.allclose(ana, num, rtol=1e-5, atol=1e-6 * scale), (key, np.abs(ana - num).max())


def test_single_expert_backward_matches_torch_autograd():
    """E = k = 1: the gate is 1 and the layer is a plain 2-layer FFN; its
    gradients are torch's autograd of that FFN (CPU float64)."""
    for ffn in ("relu", "swiglu"):
        cfg = _cfg(tokens=9, d_model=6, n_experts=1, d_hidden=10, top_k=1, ffn=ffn, noisy=False)
        inp = _np_inputs(cfg, 3)
        dy = make_upstream(cfg, seed=3).double().numpy()
        bw = oracle.backward(inp, cfg, dy, 0.0, 0.0)
        x = torch.tensor(inp["x"], requires_grad=True)
        w1 = torch.tensor(inp["w1"][0], requires_grad=True)
        w2 = torch.tensor(inp["w2"][0], requires_grad=True)
        if ffn == "relu":
            y = torch.relu(x @ w1.T) @ w2.T
            leaves = [x, w1, w2]
        else:
            w3 = torch.tensor(inp["w3"][0], requires_grad=True)
            y = (torch.nn.functional.silu(x @ w1.T) * (x @ w3.T)) @ w2.T
            leaves = [x, w1, w2, w3]
        y.backward(torch.tensor(dy))
        assert np.allclose(bw["dx"], x.grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(bw["dw1"][0], w1.grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(bw["dw2"][0], w2.grad.numpy(), rtol=1e-12, atol=1e-12)
        if ffn == "swiglu":
            assert np.allclose(bw["dw3"][0], leaves[3].grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(bw["dw_gate"], 0.0) and np.allclose(bw["dbias"], 0.0)


def test_dense_mixture_backward_matches_torch_autograd():
    """k = E without noise: y = sum_e softmax(x W_g^T + b)_e E_e(x), the
    textbook dense mixture; gradients of sum(dy * y) from torch autograd."""
    cfg = _cfg(tokens=8, d_model=6, n_experts=4, d_hidden=5, top_k=4, noisy=False)
    inp = _np_inputs(cfg, 5)
    inp["bias"] = np.array([0.3, -0.2, 0.1, 0.0])
    dy = make_upstream(cfg, seed=5).double().numpy()
    bw = oracle.backward(inp, cfg, dy, 0.0, 0.0)
    x = torch.tensor(inp["x"], requires_grad=True)
    wg = torch.tensor(inp["w_gate"], requires_grad=True)
    b = torch.tensor(inp["bias"], requires_grad=True)
    w1 = torch.tensor(inp["w1"], requires_grad=True)
    w2 = torch.tensor(inp["w2"], requires_grad=True)
    P = torch.softmax(x @ wg.T + b, dim=1)
    y = sum(P[:, e:e + 1] * (torch.relu(x @ w1[e].T) @ w2[e].T) for e in range(4))
    y.backward(torch.tensor(dy))
    for ours, ref in ((bw["dx"], x), (bw["dw_gate"], wg), (bw["dbias"], b), (bw["dw1"], w1),
                      (bw["dw2"], w2)):
        assert np.allclose(ours, ref.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_cv_squared_gradient_closed_forms():
    """CV^2([a, b]) = ((a - b) / (a + b))^2, so d/da = 4 b (a - b) / (a + b)^3;
    CV^2 is scale invariant, so sum_i v_i dCV^2/dv_i = 0; zero mean gives 0."""
    a, b = 3.0, 1.25
    g = oracle.cv_squared_grad([a, b])
    assert g[0] == pytest.approx(4 * b * (a - b) / (a + b) ** 3, rel=1e-14)
    assert g[1] == pytest.approx(4 * a * (b - a) / (a + b) ** 3, rel=1e-14)
    v = np.random.default_rng(0).uniform(0.5, 4.0, 37)
    assert abs(float(v @ oracle.cv_squared_grad(v))) < 1e-14
    assert (oracle.cv_squared_grad(np.zeros(5)) == 0).all()
    assert (oracle.cv_squared_grad(np.full(6, 2.5)) == 0).all()


def test_softmax_gradient_is_shift_invariant():
    """Without noise and balance losses, adding a constant to every score of a
    token leaves the gates unchanged, so the score gradients of each token sum
    to zero, and so do the bias gradients."""
    cfg = _cfg(tokens=40, d_model=8, n_experts=9, d_hidden=6, top_k=3, noisy=False)
    inp = _np_inputs(cfg, 7)
    dy = make_upstream(cfg, seed=7).double().numpy()
    bw = oracle.backward(inp, cfg, dy, 0.0, 0.0)
    assert np.allclose(bw["dH"].sum(axis=1), 0.0, atol=1e-13)
    assert abs(bw["dbias"].sum()) < 1e-12
    # dropped experts get no score gradient from the combine
    G = oracle.dense_gates(bw["forward"]["idx"], bw["forward"]["gates"], cfg.n_experts)
    assert (bw["dH"][G == 0] == 0).all()


def test_rank_experts_follow_the_tie_break():
    H = np.array([[1.0, 3.0, 3.0, 0.5, 3.0], [0.0, 0.0, 0.0, 0.0, 0.0]])
    jk, jk1 = oracle.rank_experts(H, 2)
    assert jk.tolist() == [2, 1] and jk1.tolist() == [4, 2]
    jk, jk1 = oracle.rank_experts(H, 5)
    assert jk.tolist() == [3, 4] and jk1.tolist() == [-1, -1]


def test_expert_backward_matches_torch_on_random_rows():
    """The per-expert backward (ReLU and SwiGLU) equals torch autograd on
    random rows, tables and output gradients (CPU float64)."""
    rng = np.random.default_rng(2)
    X = rng.standard_normal((11, 6))
    w1, w3, w2 = rng.standard_normal((9, 6)), rng.standard_normal((9, 6)), rng.standard_normal((6, 9))
    dY = rng.standard_normal((11, 6))
    tX, t1, t3, t2 = (torch.tensor(a, requires_grad=True) for a in (X, w1, w3, w2))
    (torch.relu(tX @ t1.T) @ t2.T).backward(torch.tensor(dY))
    dX, dW1, dW2 = oracle.expert_relu_backward(X, w1, w2, dY)
    for ours, ref in ((dX, tX), (dW1, t1), (dW2, t2)):
        assert np.allclose(ours, ref.grad.numpy(), rtol=1e-12, atol=1e-12)
    tX, t1, t3, t2 = (torch.tensor(a, requires_grad=True) for a in (X, w1, w3, w2))
    ((torch.nn.functional.silu(tX @ t1.T) * (tX @ t3.T)) @ t2.T).backward(torch.tensor(dY))
    dX, dW1, dW3, dW2 = oracle.expert_swiglu_backward(X, w1, w3, w2, dY)
    for ours, ref in ((dX, tX), (dW1, t1), (dW3, t3), (dW2, t2)):
        assert np.allclose(ours, ref.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_normal_pdf_and_sigmoid_closed_forms():
    assert oracle.normal_pdf(0.0) == pytest.approx(1.0 / math.sqrt(2 * math.pi), rel=1e-15)
    z = np.linspace(-5, 5, 101)
    # phi is the derivative of Phi (central difference of the pinned CDF)
    h = 1e-5
    num = (oracle.normal_cdf(z + h) - oracle.normal_cdf(z - h)) / (2 * h)
    assert np.allclose(oracle.normal_pdf(z), num, rtol=1e-7, atol=1e-10)
    assert np.allclose(oracle.sigmoid(z), 1.0 / (1.0 + np.exp(-z)), rtol=1e-14)


HIER_FD_CASES = [
    dict(ffn="relu", noisy=True, wi=0.7, wl=1.0),
    dict(ffn="swiglu", noisy=False, wi=1.1, wl=0.0),
    dict(ffn="relu", noisy=True, wi=0.0, wl=0.0, k_groups=1, k_per_group=3),
    dict(ffn="relu", noisy=True, wi=0.5, wl=0.0, k_groups=3, k_per_group=1, capacity=3),
]


def _hier_cfg(**kw):
    base = dict(name="bwh", tokens=6, d_model=5, n_experts=12, d_hidden=7, noisy=True,
                dtype="f32", gate_std=0.6, n_groups=3, k_groups=2, k_per_group=2)
    base.update(kw)
    base["top_k"] = base["k_groups"] * base["k_per_group"]
    return MoEConfig(**base)


@pytest.mark.parametrize("case", HIER_FD_CASES,
                         ids=lambda c: "-".join(f"{k}={v}" for k, v in c.items()))
def test_hier_gradients_match_central_differences(case):
    """The hierarchy: every gradient, both levels' tables included, equals
    the central difference of the oracle's forward objective (whose hard
    load does not move under a small perturbation)."""
    case = dict(case)
    wi, wl = case.pop("wi"), case.pop("wl")
    cfg = _hier_cfg(**case)
    for seed in range(80):
        inp = _np_inputs(cfg, seed)
        if _min_margin(inp, cfg) > 5e-3:
            break
    else:
        pytest.fail("no seed with well-separated scores")
    dy = make_upstream(cfg, seed=seed).double().numpy()
    bw = oracle.backward(inp, cfg, dy, wi, wl)
    assert bw["dbias"] is None
    h = 1e-6
    names = [("x", "dx"), ("w_gate", "dw_gate"), ("w_gate_p", "dw_gate_p"), ("w1", "dw1"),
             ("w2", "dw2")]
    if cfg.noisy:
        names += [("w_noise", "dw_noise"), ("w_noise_p", "dw_noise_p")]
    if cfg.ffn == "swiglu":
        names.append(("w3", "dw3"))
    for key, gkey in names:
        base = inp[key]
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            old = base[i]
            base[i] = old + h
            fp = _objective(inp, cfg, dy, wi, wl)
            base[i] = old - h
            fm = _objective(inp, cfg, dy, wi, wl)
            base[i] = old
            num[i] = (fp - fm) / (2 * h)
        ana = bw[gkey]
        scale = max(1.0, np.abs(num).max())
        assert np.allclose(ana, num, rtol=1e-5, atol=1e-6 * scale), (key, np.abs(ana - num).max())


def test_hier_with_one_group_is_the_flat_gate():
    """One group kept out of one: the primary gate is 1 and has no gradient,
    and the layer is the flat gate over the group's experts, so every
    gradient equals the flat backward's (load weight 0: the hierarchy's load
    is a hard count, the flat noisy gate's a smooth estimate)."""
    for noisy in (True, False):
        hcfg = _hier_cfg(n_groups=1, k_groups=1, k_per_group=2, n_experts=5, noisy=noisy)
        inp = _np_inputs(hcfg, 4)
        fcfg = _cfg(n_experts=5, top_k=2, noisy=noisy)
        finp = dict(inp, bias=np.zeros(5), eps=None if inp["eps"] is None else inp["eps"][:, 0, :])
        dy = make_upstream(hcfg, seed=4).double().numpy()
        hb = oracle.backward(inp, hcfg, dy, 0.6, 0.0)
        fb = oracle.backward(finp, fcfg, dy, 0.6, 0.0)
        for key in ("dx", "dw_gate", "dw_noise", "dw1", "dw2"):
            if fb[key] is None:
                assert hb[key] is None
                continue
            assert np.allclose(hb[key], fb[key], rtol=1e-12, atol=1e-12), key
        assert np.allclose(hb["dw_gate_p"], 0.0, atol=1e-12)
        if noisy:
            assert np.allclose(hb["dw_noise_p"], 0.0, atol=1e-12)
