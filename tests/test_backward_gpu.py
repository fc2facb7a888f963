"""Parity of the HIP backward pass (moe_backward through the C ABI) with the
CPU oracle's backward, on seeded inputs whose scores are well separated.

Bar: every gradient element within |g - g_ref| <= rtol |g_ref| + rtol rms,
rms the larger of the whole tensor's and that of the element's slice along
the leading axis (the token of a dx row, the expert of a table gradient: an
expert with many rows sums larger terms that cancel), rtol 3e-2 for bf16
layers (derived below) and 1e-4 for fp32 layers, plus a relative Frobenius
error below 1e-2 (bf16) or 5e-5 (fp32).  In bf16 the forward's expert outputs are stored in bf16 (relative
error about 2^-9), and the gate gradient reads them: the error of each
token's gate gradient is set by that token's scale, so a rarely used expert,
whose table-gradient row is small, still carries errors of the global size.
The kept experts, and the experts ranked k-1, k, k+1 and k+2, must not
change under rounding: inputs are drawn from the first seed whose
consecutive sorted scores (oracle, fp64) around the threshold all differ by
at least 1e-5 (fp32 scores differ from fp64 ones by about 1e-7).  Repeated calls must give bitwise identical results."""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_check import np_
from sparsely_gated_mixture_noisy_amd import _lib as L
from sparsely_gated_mixture_noisy_amd.inputs import CONFIGS, make_inputs, make_upstream

pytestmark = pytest.mark.gpu

# bf16: about three bf16 roundings meet on each product path (the gate-scaled
# output gradient or the hidden gradient as an operand, the recomputed hidden
# activation, the stored result), each with relative error up to 2^-9, so an
# element's error has sigma of about sqrt(3) * 2^-9 * rms = 3.4e-3 rms; 3e-2
# keeps the elementwise bar near 9 sigma over 1e8 elements, while the
# Frobenius bound (1e-2; observed about 3e-3) stays tight.
RTOL = {"bf16": 3e-2, "f32": 1e-4}
FRO = {"bf16": 1e-2, "f32": 5e-5}
GAP = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _separated(ref, k):
    """Consecutive sorted noisy scores around ranks k-1 .. k+2 differ by GAP
    (the hierarchy, which has no smooth load: the k-th and (k+1)-th scores
    of both levels)."""
    if "H" not in ref["gate_info"]:
        return bool((ref["margin"] >= GAP).all())
    H = ref["gate_info"]["H"]
    srt = -np.sort(-H, axis=1)
    E = H.shape[1]
    lo, hi = max(0, k - 2), min(E - 1, k + 1)
    if hi <= lo:
        return True
    gaps = srt[:, lo:hi] - srt[:, lo + 1:hi + 1]
    return bool((gaps >= GAP).all())


def _inputs(cfg, seed0=0):
    for seed in range(seed0, seed0 + 20):
        inp = make_inputs(cfg, seed=seed, device="cuda")
        cpu = {key: (v.to("cpu") if v is not None else None) for key, v in inp.items()}
        ref = oracle.forward(cpu, cfg, with_experts=False)
        if cfg.tokens == 0 or _separated(ref, cfg.top_k):
            return seed, inp, cpu
    pytest.fail("no seed with separated scores")


def _check(name, got, ref, rtol, fro_max):
    got = np_(got).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if ref.size == 0:
        return
    rms_all = np.sqrt(np.mean(ref * ref))
    if ref.ndim > 1:
        rms = np.sqrt(np.mean((ref * ref).reshape(ref.shape[0], -1), axis=1))
        rms = np.maximum(rms, rms_all).reshape((-1,) + (1,) * (ref.ndim - 1))
    else:
        rms = np.full(ref.shape, rms_all)
    err = np.abs(got - ref)
    bound = rtol * np.abs(ref) + rtol * rms
    worst = float(np.max(err - bound))
    assert worst <= 0, f"{name}: max excess {worst:.3e} (max err {err.max():.3e})"
    fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert fro <= fro_max, f"{name}: relative Frobenius error {fro:.3e}"


CASES = {
    "tiny": (CONFIGS["tiny"], 0.7, 1.3),
    "tiny_ragged_swiglu": (CONFIGS["tiny"].replace(tokens=77, ffn="swiglu"), 0.5, 0.8),
    "tiny_noise_free": (CONFIGS["tiny"].replace(tokens=90, noisy=False), 1.0, 0.0),
    # fp32, two expert blocks of 256 in the gate tiles: the rank kernel, then
    # the gradient kernel
    "tiny_e300": (CONFIGS["tiny"].replace(tokens=120, n_experts=300), 0.6, 1.2),
    "bf16_relu": (CONFIGS["flat256"].replace(tokens=400, n_experts=24, d_model=128, d_hidden=256),
                  0.6, 1.1),
    "bf16_swiglu": (CONFIGS["flat256"].replace(tokens=300, n_experts=12, d_model=128,
                                               d_hidden=192, ffn="swiglu", top_k=2), 0.4, 0.9),
    # experts averaging about 17 rows: 32-row tiles of the three-product
    # SwiGLU recompute and of dX, a ragged last column tile (192 hidden units)
    "bf16_swiglu_small_experts": (CONFIGS["flat256"].replace(tokens=200, n_experts=24, d_model=128,
                                                             d_hidden=192, ffn="swiglu", top_k=2),
                                  0.4, 0.9),
    # two expert blocks in the gate tiles, a bias, a ragged last tile, idle experts
    "bf16_e300_bias": (CONFIGS["zipf2048"].replace(tokens=230, n_experts=300, d_model=64,
                                                   d_hidden=128), 0.3, 2.0),
    # three expert blocks in the gate tiles: a ragged last tile (333 = 10 x 32
    # + 13) and a part-filled last block (600 = 2 x 256 + 88)
    "bf16_e600_three_blocks": (CONFIGS["zipf2048"].replace(tokens=333, n_experts=600,
                                                           d_model=128, d_hidden=64),
                               0.4, 1.5),
    "bf16_noise_free_k3": (CONFIGS["flat256"].replace(tokens=260, n_experts=10, d_model=192,
                                                      d_hidden=320, noisy=False, top_k=3),
                           1.2, 0.0),
    "bf16_flat256_t512": (CONFIGS["flat256"].replace(tokens=512), 1.0, 1.0),
    # experts capped at 6 rows: dropped slots add nothing to y or dx
    "bf16_capacity6": (CONFIGS["flat256"].replace(tokens=300, n_experts=24, d_model=128,
                                                  d_hidden=256, capacity=6), 0.7, 1.2),
    "tiny_capacity40": (CONFIGS["tiny"].replace(capacity=40), 0.5, 0.5),
    # the hierarchy: both levels' tables, noisy and noise-free, a capacity
    "tiny_hier": (CONFIGS["tiny"].replace(tokens=150, n_experts=12, n_groups=4, k_groups=2,
                                          k_per_group=1, top_k=2), 0.9, 1.0),
    "tiny_hier_swiglu_noise_free": (CONFIGS["tiny"].replace(tokens=97, n_experts=12, n_groups=3,
                                                            k_groups=1, k_per_group=2, top_k=2,
                                                            ffn="swiglu", noisy=False), 1.0, 0.0),
    "bf16_hier": (CONFIGS["hier4096"].replace(tokens=300, n_experts=64, d_model=128,
                                              d_hidden=256), 0.8, 1.0),
    "bf16_hier_capacity10": (CONFIGS["hier4096"].replace(tokens=400, n_experts=64, d_model=128,
                                                         d_hidden=256, capacity=10), 0.8, 0.0),
    # experts with >= 256 rows on average: the large-tile products (ragged
    # last column tiles; at h = 8192 the XCD-grouped order for the hidden
    # layer, dHid and dW2, and the swapped enumeration for dW1 and dW3)
    "bf16_big_relu": (CONFIGS["flat256"].replace(tokens=700, n_experts=4, d_model=256,
                                                 d_hidden=640, top_k=2), 0.8, 1.0),
    "bf16_big_swiglu": (CONFIGS["mixtral"].replace(tokens=600, n_experts=4, d_model=256,
                                                   d_hidden=320), 0.8, 0.0),
    "bf16_big_swiglu_h8192": (CONFIGS["mixtral"].replace(tokens=600, n_experts=4, d_model=64,
                                                         d_hidden=8192), 0.8, 0.0),
    # the large-tile backward on capped experts (about 300 rows each, 200 kept)
    "bf16_big_swiglu_cap200": (CONFIGS["mixtral"].replace(tokens=600, n_experts=4, d_model=256,
                                                          d_hidden=320, capacity=200), 0.8, 0.0),
    # large-tile path with a Zipf bias: an idle expert (zero table gradients),
    # experts with 1 to 4 rows (mostly zero-row positions) and one of 2342 rows
    "bf16_big_zipf_idle": (CONFIGS["zipf2048"].replace(tokens=3100, n_experts=12, d_model=64,
                                                       d_hidden=128, top_k=1), 0.5, 0.5),
    # 15 rows per expert on average (table gradients on one LDS buffer), idle
    # experts, and nine experts with 65 to 463 rows: tiles of several K slices
    # with a ragged last slice
    "bf16_zipf_one_buffer": (CONFIGS["zipf2048"].replace(tokens=1200, n_experts=160, d_model=64,
                                                         d_hidden=128), 0.5, 0.5),
    # d_model 512 ReLU: the hidden layer on the fused per-tile kernel.  About
    # 250 rows per expert: three tiles each (96, 96 and 58 rows: two and three
    # 32-row blocks, a ragged last block), four hidden chunks
    "bf16_d512_three_tiles": (CONFIGS["flat256"].replace(tokens=1000, n_experts=8, top_k=2),
                              0.6, 1.1),
    # the same kernel with two hidden chunks, a Zipf bias: idle experts,
    # single-row experts and hot experts of several tiles
    "bf16_d512_zipf_h512": (CONFIGS["zipf2048"].replace(tokens=700, n_experts=48, d_hidden=512),
                            0.5, 0.9),
    # one group, then one expert: both softmax levels are a single weight of 1
    "bf16_hier_k1": (CONFIGS["hier4096"].replace(tokens=200, n_experts=64, d_model=128,
                                                 d_hidden=256, k_groups=1, k_per_group=1,
                                                 top_k=1), 0.7, 0.0),
}
KEYS = ("dx", "dw_gate", "dw_noise", "dbias", "dw1", "dw3", "dw2", "dw_gate_p", "dw_noise_p")


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    cfg, wi, wl = CASES[name]
    seed, inp, cpu = _inputs(cfg)
    _say(f"[backward] {name} seed {seed} T={cfg.tokens} E={cfg.n_experts} d={cfg.d_model} "
         f"h={cfg.d_hidden} k={cfg.top_k} {cfg.ffn} {cfg.dtype} noisy={cfg.noisy}")
    dy = make_upstream(cfg, seed=seed, device="cuda")
    fwd = L.forward(cfg, inp["x"], inp, inp, wi, wl, balance=True, save=True)
    g1 = L.backward(cfg, inp["x"], inp, inp, fwd, dy, wi, wl)
    torch.cuda.synchronize()
    ref = oracle.backward(cpu, cfg, dy.to("cpu"), wi, wl)
    assert (np_(fwd.topk_idx) == ref["forward"]["idx"]).all()
    rtol = RTOL[cfg.dtype]
    for key in KEYS:
        got = getattr(g1, key)
        if got is None:
            assert ref.get(key) is None, key
            continue
        _check(key, got, ref[key], rtol, FRO[cfg.dtype])
    # deterministic: a second call gives the same bits
    g2 = L.backward(cfg, inp["x"], inp, inp, fwd, dy, wi, wl)
    torch.cuda.synchronize()
    for key in KEYS:
        a, b = getattr(g1, key), getattr(g2, key)
        if a is not None:
            assert torch.equal(a, b), f"{key} differs between two calls"


@pytest.mark.parametrize("name", ["bf16_d512_three_tiles", "bf16_d512_zipf_h512"])
def test_backward_packed_tables_match_plain(name):
    """With the forward's packed expert tables the backward reads W1 from
    them (the fused hidden-layer kernel): the same values in the same order,
    so every gradient is bitwise equal to the plain-table call's."""
    cfg, wi, wl = CASES[name]
    seed, inp, _ = _inputs(cfg)
    _say(f"[backward] packed against plain tables: {name} seed {seed}")
    dy = make_upstream(cfg, seed=seed, device="cuda")
    binp = L.packed_params(cfg, inp)
    assert binp.get("w_packed") is not None
    fwd = L.forward(cfg, inp["x"], inp, inp, wi, wl, balance=True, save=True)
    g_plain = L.backward(cfg, inp["x"], inp, inp, fwd, dy, wi, wl)
    g_packed = L.backward(cfg, inp["x"], binp, binp, fwd, dy, wi, wl)
    torch.cuda.synchronize()
    for key in KEYS:
        a, b = getattr(g_plain, key), getattr(g_packed, key)
        if a is not None:
            assert torch.equal(a, b), f"{key} differs between packed and plain tables"


@pytest.mark.parametrize("base", ["flat256", "hier4096"])
def test_backward_empty_batch_and_idle_experts(base):
    """T = 0: dx is empty and every table gradient is zero."""
    cfg = CONFIGS[base].replace(tokens=0, n_experts=32, d_model=64, d_hidden=128)
    inp = make_inputs(cfg, seed=0, device="cuda")
    dy = make_upstream(cfg, seed=0, device="cuda")
    fwd = L.forward(cfg, inp["x"], inp, inp, 1.0, 1.0, balance=True, save=True)
    g = L.Grads(cfg, 0, "cuda")
    keys = [key for key in KEYS if key != "dx" and getattr(g, key) is not None]
    for key in keys:
        getattr(g, key).fill_(7.0)
    L.Backward(cfg, inp["x"], inp, inp, fwd, dy, 1.0, 1.0, grads=g)()
    torch.cuda.synchronize()
    for key in keys:
        assert (getattr(g, key) == 0).all(), key


def test_backward_rejects_missing_and_misplaced_inputs():
    hier = CONFIGS["hier4096"].replace(tokens=64, n_experts=64, d_model=64, d_hidden=128)
    assert L.backward_workspace_size(hier) > 0
    hinp = make_inputs(hier, seed=0, device="cuda")
    hdy = make_upstream(hier, seed=0, device="cuda")
    hfwd = L.forward(hier, hinp["x"], hinp, hinp, 1.0, 1.0, balance=True, save=True)
    # the hierarchy has no bias, so no bias gradient
    g = L.Grads(hier, 64, "cuda")
    g.dbias = torch.empty(hier.n_experts, dtype=torch.float32, device="cuda")
    with pytest.raises(L.MoEError) as e:
        L.Backward(hier, hinp["x"], hinp, hinp, hfwd, hdy, grads=g)()
    assert e.value.status == L.MOE_ERR_INVALID_ARG
    flat = CONFIGS["flat256"].replace(tokens=64, n_experts=8, d_model=64, d_hidden=128)
    inp = make_inputs(flat, seed=0, device="cuda")
    dy = make_upstream(flat, seed=0, device="cuda")
    fwd = L.forward(flat, inp["x"], inp, inp, 1.0, 1.0, balance=True, save=False)
    with pytest.raises(L.MoEError) as e:
        L.backward(flat, inp["x"], inp, inp, fwd, dy)
    assert e.value.status == L.MOE_ERR_INVALID_ARG
    # the primary tables' gradients belong to the hierarchy
    sfwd = L.forward(flat, inp["x"], inp, inp, 1.0, 1.0, balance=True, save=True)
    g = L.Grads(flat, 64, "cuda")
    g.dw_gate_p = torch.empty((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.MoEError) as e:
        L.Backward(flat, inp["x"], inp, inp, sfwd, dy, grads=g)()
    assert e.value.status == L.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["flat256", "zipf2048"])
def test_backward_flat_full_size_sampled(name):
    """The full flat layers in the launch configuration the timings use: the
    paper-shaped one (8192 tokens, 256 experts, 512 -> 1024 -> 512, k = 4,
    noisy) and the Zipf-biased one (32768 tokens, 2048 experts, k = 2: idle,
    single-row and hot experts of many tiles).  The oracle computes, one by
    one: the table gradients of sampled experts (from those experts' rows
    only; the hottest expert is always among them) and the input gradients
    of sampled tokens (from their own slots; the load-loss and importance
    gradients need only the per-expert statistics, which the oracle computes
    over all tokens).  Tokens whose scores around the threshold are within
    1e-5 are not sampled, nor experts that hold such a token in either
    routing."""
    cfg = CONFIGS[name]
    wi, wl = 1.0, 1.0
    inp = make_inputs(cfg, seed=0, device="cuda")
    cpu = {key: (v.to("cpu") if v is not None else None) for key, v in inp.items()}
    dy = make_upstream(cfg, seed=0, device="cuda")
    _say(f"[backward] {name} full size: forward + backward on the GPU")
    binp = L.packed_params(cfg, inp)
    fwd = L.forward(cfg, inp["x"], binp, binp, wi, wl, balance=True, save=True)
    g = L.backward(cfg, inp["x"], binp, binp, fwd, dy, wi, wl)
    torch.cuda.synchronize()
    _say("[backward] oracle gate and statistics")
    x = cpu["x"].double().numpy()
    dyn = dy.to("cpu").double().numpy()
    gi = oracle.gate(cpu, cfg)
    T, k, E = cfg.tokens, cfg.top_k, cfg.n_experts
    idx, gates = gi["idx"], gi["gates"]
    srt = -np.sort(-gi["H"], axis=1)
    risky = ((srt[:, k - 2:k + 1] - srt[:, k - 1:k + 2]) < GAP).any(axis=1)
    gidx = np_(fwd.topk_idx)
    assert (gidx[~risky] == idx[~risky]).all()
    counts, offsets, perm, inv = oracle.route(idx, E)
    imp = oracle.importance(idx, gates, E)
    load = oracle.load_estimate(gi["clean"], gi["sp"], gi["H"], idx, gi["kth"], gi["k1th"])
    dimp = wi * oracle.cv_squared_grad(imp)
    w1 = cpu["w1"].double().numpy()
    w2 = cpu["w2"].double().numpy()
    rng = np.random.default_rng(1)

    # table gradients of sampled experts
    risky_e = set(idx[risky].reshape(-1).tolist()) | set(gidx[risky].reshape(-1).tolist())
    cand = [e for e in range(E) if e not in risky_e and counts[e] > 0]
    hot = max(cand, key=lambda e: counts[e])
    sample = [hot] + [e for e in rng.choice(cand, size=6, replace=False) if e != hot][:5]
    for e in sample:
        rows = perm[offsets[e]:offsets[e + 1]]
        toks = rows // k
        dY = gates.reshape(-1)[rows][:, None] * dyn[toks]
        _, dw1, dw2 = oracle.expert_relu_backward(x[toks], w1[e], w2[e], dY)
        _check(f"dw1[{e}]", g.dw1[e], dw1, RTOL["bf16"], FRO["bf16"])
        _check(f"dw2[{e}]", g.dw2[e], dw2, RTOL["bf16"], FRO["bf16"])

    # input gradients of sampled tokens: the expert part from each kept
    # expert's own backward, the gate part from the oracle's flat-gate
    # backward on the sampled tokens, given their gate gradients and the
    # whole layer's load (whose CV^2 gradient spans every token)
    toks = np.sort(rng.choice(np.nonzero(~risky)[0], size=24, replace=False))
    dgate = np.zeros((toks.size, k))
    dxe = np.zeros((toks.size, cfg.d_model))
    for n, t in enumerate(toks):
        xt = x[t:t + 1]
        for s in range(k):
            e = idx[t, s]
            dgate[n, s] = oracle.expert_relu(xt, w1[e], w2[e])[0] @ dyn[t] + dimp[e]
            dX, _, _ = oracle.expert_relu_backward(xt, w1[e], w2[e], gates[t, s] * dyn[t:t + 1])
            dxe[n] += dX[0]
    sub_gate = {key: gi[key][toks] for key in ("clean", "sp", "H", "kth", "k1th")}
    sub_fw = dict(gate_info=sub_gate, idx=idx[toks], gates=gates[toks], load=load)
    sub_inp = dict(eps=cpu["eps"][toks], w_gate=cpu["w_gate"], w_noise=cpu["w_noise"])
    res = oracle.moe_oracle._flat_gate_backward(sub_inp, cfg.replace(tokens=toks.size), x[toks],
                                                sub_fw, dgate, wl)
    dx_ref = dxe + res["dx"]
    got = np_(g.dx)[toks]
    _check("dx[sampled]", got, dx_ref, RTOL["bf16"], FRO["bf16"])


def test_backward_mixtral_full_size_sampled():
    """The Mixtral-shaped layer (8192 tokens, 8 SwiGLU experts 4096 -> 14336
    -> 4096, top-2, noise-free) in the launch configuration the timings use,
    where the hidden layer runs on the large-tile GEMM.  The oracle computes,
    one by one: for sampled experts and hidden units, the rows of dW1 and dW3
    and the columns of dW2 of those units (hidden units are independent, so
    the unit-sliced expert gives them exactly), and the input gradients of
    sampled tokens (their own slots and the gate part)."""
    cfg = CONFIGS["mixtral"]
    wi, wl = 1.0, 0.0
    inp = make_inputs(cfg, seed=0, device="cuda")
    dy = make_upstream(cfg, seed=0, device="cuda")
    _say("[backward] mixtral full size: forward + backward on the GPU")
    binp = L.packed_params(cfg, inp)
    fwd = L.forward(cfg, inp["x"], binp, binp, wi, wl, balance=True, save=True)
    g = L.backward(cfg, inp["x"], binp, binp, fwd, dy, wi, wl)
    torch.cuda.synchronize()
    _say("[backward] oracle gate and statistics")
    big = ("w1", "w2", "w3")
    cpu = {key: (v.to("cpu") if v is not None else None) for key, v in inp.items()
           if key not in big}
    x = cpu["x"].double().numpy()
    dyn = dy.to("cpu").double().numpy()
    gi = oracle.gate(cpu, cfg)
    T, k, E = cfg.tokens, cfg.top_k, cfg.n_experts
    idx, gates = gi["idx"], gi["gates"]
    assert (np_(fwd.topk_idx) == idx).all()
    counts, offsets, perm, inv = oracle.route(idx, E)
    dimp = wi * oracle.cv_squared_grad(oracle.importance(idx, gates, E))

    def tables(e):
        return tuple(inp[key][e].to("cpu").double().numpy() for key in ("w1", "w3", "w2"))

    rng = np.random.default_rng(1)
    # table gradients of sampled experts and hidden units
    for e in rng.choice(np.nonzero(counts > 0)[0], size=2, replace=False):
        w1e, w3e, w2e = tables(e)
        rows = perm[offsets[e]:offsets[e + 1]]
        toks = rows // k
        dY = gates.reshape(-1)[rows][:, None] * dyn[toks]
        units = np.sort(rng.choice(cfg.d_hidden, size=8, replace=False))
        _, dw1, dw3, dw2 = oracle.expert_swiglu_backward(x[toks], w1e[units], w3e[units],
                                                         w2e[:, units], dY)
        _check(f"dw1[{e}][units]", g.dw1[e][torch.from_numpy(units).cuda()], dw1,
               RTOL["bf16"], FRO["bf16"])
        _check(f"dw3[{e}][units]", g.dw3[e][torch.from_numpy(units).cuda()], dw3,
               RTOL["bf16"], FRO["bf16"])
        _check(f"dw2[{e}][:, units]", g.dw2[e][:, torch.from_numpy(units).cuda()], dw2,
               RTOL["bf16"], FRO["bf16"])

    # input gradients of sampled tokens: expert part + gate part
    srt = -np.sort(-gi["H"], axis=1)
    risky = ((srt[:, k - 2:k + 1] - srt[:, k - 1:k + 2]) < GAP).any(axis=1)
    toks = np.sort(rng.choice(np.nonzero(~risky)[0], size=12, replace=False))
    dxe = np.zeros((toks.size, cfg.d_model))
    dg = np.zeros((toks.size, k))
    for e in np.unique(idx[toks]):
        w1e, w3e, w2e = tables(e)
        for n, t in enumerate(toks):
            for sl in np.nonzero(idx[t] == e)[0]:
                xt = x[t:t + 1]
                dg[n, sl] = oracle.expert_swiglu(xt, w1e, w3e, w2e)[0] @ dyn[t] + dimp[e]
                dX, _, _, _ = oracle.expert_swiglu_backward(xt, w1e, w3e, w2e,
                                                            gates[t, sl] * dyn[t:t + 1])
                dxe[n] += dX[0]
    wg = cpu["w_gate"].double().numpy()
    dx_ref = np.zeros_like(dxe)
    for n, t in enumerate(toks):
        dH = np.zeros(E)
        dH[idx[t]] = gates[t] * (dg[n] - gates[t] @ dg[n])
        dx_ref[n] = dxe[n] + dH @ wg
    _check("dx[sampled]", np_(g.dx)[toks], dx_ref, RTOL["bf16"], FRO["bf16"])
    _say("[backward] mixtral full size: ok")


def test_backward_hier4096_full_size_sampled():
    """The full 4096-expert hierarchy (16384 tokens, 16 groups x 256,
    512 -> 1024 -> 512, two groups then two experts, noisy at both levels)
    in the launch configuration the timings use.  The oracle computes, one
    by one: the tables of sampled experts (expert tables from their rows; the
    secondary gate and noise rows from the tokens that keep them, through
    the oracle's own hierarchical gate backward on that sub-batch) and the
    input gradients of sampled tokens.  A token's gate gradients need the
    outputs of its k experts and the importance gradient, which the oracle
    computes over all tokens.  The primary tables' gradients sum over every
    token and so need every expert's outputs; they are checked at the
    smaller hierarchical sizes above, with the same kernels.  Tokens whose
    margin at either level is below 1e-5 are not sampled, nor experts that
    hold such a token."""
    cfg = CONFIGS["hier4096"]
    wi, wl = 1.0, 1.0
    inp = make_inputs(cfg, seed=0, device="cuda")
    cpu = {key: (v.to("cpu") if v is not None else None) for key, v in inp.items()}
    dy = make_upstream(cfg, seed=0, device="cuda")
    _say("[backward] hier4096 full size: forward + backward on the GPU")
    binp = L.packed_params(cfg, inp)
    fwd = L.forward(cfg, inp["x"], binp, binp, wi, wl, balance=True, save=True)
    g = L.backward(cfg, inp["x"], binp, binp, fwd, dy, wi, wl)
    torch.cuda.synchronize()
    _say("[backward] oracle hierarchical gate and statistics")
    x = cpu["x"].double().numpy()
    dyn = dy.to("cpu").double().numpy()
    gi = oracle.gate(cpu, cfg)
    T, k, E = cfg.tokens, cfg.top_k, cfg.n_experts
    idx, gates = gi["idx"], gi["gates"]
    risky = gi["margin"] < GAP
    assert (np_(fwd.topk_idx)[~risky] == idx[~risky]).all()
    counts, offsets, perm, inv = oracle.route(idx, E)
    dimp = wi * oracle.cv_squared_grad(oracle.importance(idx, gates, E))
    tabs = {key: cpu[key].double().numpy() for key in ("w_gate", "w_noise", "w_gate_p",
                                                      "w_noise_p")}
    eps, eps_p = cpu["eps"].double().numpy(), cpu["eps_p"].double().numpy()
    experts = {}

    def expert(e):
        if e not in experts:
            experts[e] = (cpu["w1"][e].double().numpy(), cpu["w2"][e].double().numpy())
        return experts[e]

    def gate_side(toks):
        """The oracle's hierarchical gate backward on a sub-batch of tokens."""
        dgate = np.zeros((toks.size, k))
        for n, t in enumerate(toks):
            for s in range(k):
                e = int(idx[t, s])
                w1e, w2e = expert(e)
                dgate[n, s] = oracle.expert_relu(x[t:t + 1], w1e, w2e)[0] @ dyn[t] + dimp[e]
        sub = dict(idx=idx[toks], primary=dict(gates=gi["primary"]["gates"][toks],
                                               idx=gi["primary"]["idx"][toks]))
        sinp = dict(tabs, eps=eps[toks], eps_p=eps_p[toks])
        return oracle.moe_oracle._hier_gate_backward(sinp, cfg.replace(tokens=toks.size),
                                                    x[toks], sub, dgate)

    rng = np.random.default_rng(2)
    risky_e = set(idx[risky].reshape(-1).tolist())
    cand = [e for e in range(E) if e not in risky_e and counts[e] > 0]
    _say("[backward] oracle: sampled experts")
    for e in rng.choice(cand, size=6, replace=False):
        rows = perm[offsets[e]:offsets[e + 1]]
        toks = rows // k
        w1e, w2e = expert(e)
        dY = gates.reshape(-1)[rows][:, None] * dyn[toks]
        _, dw1, dw2 = oracle.expert_relu_backward(x[toks], w1e, w2e, dY)
        _check(f"dw1[{e}]", g.dw1[e], dw1, RTOL["bf16"], FRO["bf16"])
        _check(f"dw2[{e}]", g.dw2[e], dw2, RTOL["bf16"], FRO["bf16"])
        res = gate_side(toks)
        _check(f"dw_gate[{e}]", g.dw_gate[e], res["dw_gate"][e], RTOL["bf16"], FRO["bf16"])
        _check(f"dw_noise[{e}]", g.dw_noise[e], res["dw_noise"][e], RTOL["bf16"], FRO["bf16"])

    _say("[backward] oracle: sampled tokens")
    toks = rng.choice(np.nonzero(~risky)[0], size=24, replace=False)
    dx_ref = gate_side(toks)["dx"]
    for n, t in enumerate(toks):
        for s in range(k):
            w1e, w2e = expert(int(idx[t, s]))
            dX, _, _ = oracle.expert_relu_backward(x[t:t + 1], w1e, w2e,
                                                   gates[t, s] * dyn[t:t + 1])
            dx_ref[n] += dX[0]
    _check("dx[sampled]", np_(g.dx)[toks], dx_ref, RTOL["bf16"], FRO["bf16"])
