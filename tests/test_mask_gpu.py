"""Parity of the per-batch equal-size expert mask and its threshold form
(moe_forward_mask through the C ABI) with the oracle's masked_forward.

Bar, as for the top-k layer: the kept tokens of every expert and their rows
bit-exact, the gates within 1e-5 relative, y within rtol |y_ref| + rtol
rms(y_ref) (rtol 2e-2 bf16, 1e-4 fp32), importance within 1e-5 relative and
the load (kept counts) exact.  Decisions the fp32 scores could take
differently from the fp64 oracle are excluded and counted: an expert whose
m-th and (m+1)-th best scores differ by less than 1e-4 (batch mask), or a
(token, expert) score within 1e-4 of the expert's threshold (threshold
mask); such an expert's rows are not compared, nor the tokens it keeps."""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_check import check_close, np_
from sparsely_gated_mixture_noisy_amd import _lib as L
from sparsely_gated_mixture_noisy_amd.inputs import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

MARGIN = 1e-4
RTOL = {"bf16": 2e-2, "f32": 1e-4}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cpu(inp, skip=()):
    return {k: (v.detach().cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()
            if k not in skip}


def _risky_experts(H, m, theta):
    """Experts whose kept set the fp32 scores could decide differently."""
    T, E = H.shape
    if theta is None:
        if m >= T:
            return np.zeros(E, dtype=bool)
        s = -np.sort(-H, axis=0)
        return (s[m - 1] - s[m]) < MARGIN
    return (np.abs(H - theta[None, :]) < MARGIN).any(axis=0)


def _gpu_pairs(out, T, E):
    """Dense [T][E] views of the GPU's slots: live (has a row), gate, row."""
    off = np_(out.tok_offsets)
    se, sg, sr = np_(out.slot_expert), np_(out.slot_gate), np_(out.slot_row)
    live = np.zeros((T, E), dtype=bool)
    gate = np.zeros((T, E))
    row = np.full((T, E), -1)
    for t in range(T):
        j0, j1 = off[t], off[t + 1]
        es = se[j0:j1]
        assert (np.diff(es) > 0).all(), "slots of a token in ascending expert order"
        live[t, es] = True
        gate[t, es] = sg[j0:j1]
        row[t, es] = sr[j0:j1]
    return live, gate, row


def check_mask_layer(cfg, out, ref, m, theta, y_rows=None, y_ref=None):
    """Compare one moe_forward_mask result with the oracle's masked_forward
    dict (y compared on y_rows against y_ref when given, else whole)."""
    H, T, E = ref["H"], cfg.tokens, cfg.n_experts
    risky = _risky_experts(H, m, theta)
    live_g, gate_g, row_g = _gpu_pairs(out, T, E)
    live_r = ref["pos"] >= 0
    # tokens kept by a risky expert, on either side, are not compared
    bad_t = (ref["keep"][:, risky].any(axis=1) | live_g[:, risky].any(axis=1))
    counts, offsets, perm = np_(out.counts), np_(out.offsets), np_(out.perm)
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all()
    assert (perm[offsets[-1]:] == 0).all()
    for e in np.nonzero(~risky)[0]:
        assert counts[e] == ref["counts"][e], e
        assert (perm[offsets[e]:offsets[e + 1]] == ref["perm"][ref["offsets"][e]:ref["offsets"][e + 1]]).all(), e
        # rows of the pairs of this expert, expressed in the expert's own order
        got_rows = row_g[:, e][live_g[:, e]] - offsets[e]
        want_rows = ref["pos"][:, e][live_r[:, e]] - ref["offsets"][e]
        assert (got_rows == want_rows).all(), e
    if theta is None:
        assert (counts == min(m, T)).all()
    ok = ~bad_t
    assert (live_g[ok] == live_r[ok]).all(), "kept experts of the included tokens"
    gr = ref["gates"][ok][live_r[ok]]
    gg = gate_g[ok][live_r[ok]]
    assert (np.abs(gg - gr) <= 1e-5 * np.abs(gr)).all(), f"gate rel err {np.max(np.abs(gg - gr) / gr):.3e}"
    rows = np.nonzero(ok)[0] if y_rows is None else y_rows
    yr = ref["y"] if y_ref is None else y_ref
    worst = check_close(np_(out.y)[rows] if y_rows is not None else out.y, yr,
                        RTOL[cfg.dtype], rows=None if y_rows is not None else rows)
    # no slot at all: y = 0 exactly
    empty = np.nonzero(np.diff(np_(out.tok_offsets)) == 0)[0]
    assert (np_(out.y)[empty] == 0).all()
    if out.balance is not None:
        slack = np.zeros(E)
        for t in np.nonzero(bad_t)[0]:
            slack[ref["keep"][t] | live_g[t]] += 1.0
        imp = np_(out.importance).astype(np.float64)
        assert (np.abs(imp - ref["importance"]) <= 1e-5 * ref["importance"] + 1e-5 + slack).all()
        load = np_(out.load)
        assert (load[~risky] == ref["load"][~risky]).all()
        if not bad_t.any():
            b = np_(out.balance)
            assert abs(b[0] - ref["cv2_importance"]) <= 1e-4 * abs(ref["cv2_importance"]) + 1e-7
            assert abs(b[1] - ref["cv2_load"]) <= 1e-4 * abs(ref["cv2_load"]) + 1e-7
    return int(risky.sum()), int(bad_t.sum()), worst


def _theta_between(H, m):
    """Per expert, the midpoint between the m-th and (m+1)-th best scores."""
    s = -np.sort(-H, axis=0)
    return (0.5 * (s[m - 1] + s[m])).astype(np.float32)


CASES = {
    # name: (config, m, threshold kind: None | "mid" (between the n-th and
    # (n+1)-th best, with n = the int given) | a constant)
    "tiny_batch": (CONFIGS["tiny"], 64, None),
    "tiny_threshold_capped": (CONFIGS["tiny"].replace(tokens=200), 30, ("mid", 45)),
    "tiny_swiglu_batch": (CONFIGS["tiny"].replace(tokens=90, ffn="swiglu", noisy=False), 20, None),
    "flat256_t1000_batch": (CONFIGS["flat256"].replace(tokens=1000), 16, None),
    "flat256_t1000_threshold": (CONFIGS["flat256"].replace(tokens=1000), 40, 1.2),
    "zipf_e2048_batch": (CONFIGS["zipf2048"].replace(tokens=2000), 2, None),
    "swiglu_bf16_batch": (CONFIGS["mixtral"].replace(tokens=200, d_model=512, d_hidden=1536), 50,
                          None),
    # E * m >= 256 * E: the large-tile grouped GEMMs
    "big_relu_batch": (CONFIGS["flat256"].replace(tokens=1500, d_model=256, d_hidden=512,
                                                  n_experts=4), 700, None),
    # every expert keeps every token: the full softmax mixture
    "tiny_every_token": (CONFIGS["tiny"].replace(tokens=50), 50, None),
    # one expert keeps one token: most tokens have no expert (y = 0)
    "flat_sparse_m1": (CONFIGS["flat256"].replace(tokens=300, n_experts=64), 1, None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mask_layer_matches_oracle(name):
    cfg, m, kind = CASES[name]
    _say(f"[mask] {name}: m={m} kind={kind} {cfg}")
    inp = make_inputs(cfg, seed=0, device="cuda")
    cpu = _cpu(inp)
    H = oracle.noisy_logits(cpu["x"], cpu["w_gate"], cpu.get("w_noise"), cpu.get("bias"),
                            cpu.get("eps"))[2]
    theta = None
    if isinstance(kind, tuple):
        theta = _theta_between(H, kind[1])
    elif kind is not None:
        theta = np.full(cfg.n_experts, kind, dtype=np.float32)
    binp = L.packed_params(cfg, inp)
    th = torch.from_numpy(theta).cuda() if theta is not None else None
    out = L.forward_mask(cfg, inp["x"], binp, binp, m, th)
    torch.cuda.synchronize()
    ref = oracle.masked_forward(cpu, cfg.replace(capacity=m if theta is not None else 0),
                                rows_per_expert=m, thresholds=theta)
    nr, nt, worst = check_mask_layer(cfg, out, ref, m, theta)
    # repeated calls: the same bits
    out2 = L.forward_mask(cfg, inp["x"], binp, binp, m, th)
    torch.cuda.synchronize()
    for f in ("y", "perm", "slot_gate", "slot_row", "importance", "balance"):
        assert torch.equal(getattr(out, f), getattr(out2, f)), f
    _say(f"[mask] {name}: ok risky experts={nr} excluded tokens={nt} worst_y={worst:.2e}")


def test_mask_with_in_kernel_noise():
    """The noise drawn inside the kernels: the oracle fed its own draws."""
    seed = (0x5EED << 32) | 77
    cfg = CONFIGS["flat256"].replace(tokens=600)
    inp = make_inputs(cfg, seed=1, device="cuda")
    gen = dict(inp, eps=None, noise_seed=seed)
    out = L.forward_mask(cfg, inp["x"], gen, gen, 10)
    torch.cuda.synchronize()
    cpu = _cpu(inp)
    cpu["eps"] = oracle.draw_noise(cfg, seed)["eps"]
    ref = oracle.masked_forward(cpu, cfg, rows_per_expert=10)
    nr, nt, worst = check_mask_layer(cfg, out, ref, 10, None)
    _say(f"[mask] in-kernel noise: ok risky experts={nr} excluded tokens={nt}")


def test_mask_empty_batch():
    cfg = CONFIGS["flat256"].replace(tokens=0, n_experts=16)
    inp = make_inputs(cfg, seed=0, device="cuda")
    out = L.forward_mask(cfg, inp["x"], inp, inp, 3)
    torch.cuda.synchronize()
    assert int(np_(out.counts).sum()) == 0 and np_(out.offsets).tolist() == [0] * 17
    assert np_(out.tok_offsets).tolist() == [0]
    assert np_(out.balance).tolist() == [0.0, 0.0, 0.0]


def test_mask_rejects_bad_requests():
    cfg = CONFIGS["flat256"].replace(tokens=64, n_experts=8)
    inp = make_inputs(cfg, seed=0, device="cuda")
    for bad_cfg, m in ((cfg, 0), (cfg, 65), (cfg.replace(capacity=4), 4)):
        with pytest.raises(L.MoEError) as e:
            L.forward_mask(bad_cfg, inp["x"], inp, inp, m, ws=L.Workspace(1 << 20))
        assert e.value.status == L.MOE_ERR_INVALID_ARG


def test_mask_full_size_flat256():
    """8192 tokens, 256 experts, m = k T / E = 128 rows each: every expert's
    rows and every token's gates over the whole batch, y on sampled tokens
    (the oracle's experts one by one), the balance statistics."""
    cfg = CONFIGS["flat256"]
    m = cfg.top_k * cfg.tokens // cfg.n_experts
    inp = make_inputs(cfg, seed=0, device="cuda")
    binp = L.packed_params(cfg, inp)
    _say("[mask-full] flat256: GPU")
    out = L.forward_mask(cfg, inp["x"], binp, binp, m)
    torch.cuda.synchronize()
    _say("[mask-full] flat256: oracle mask and gates")
    cpu = _cpu(inp, skip=("w1", "w2", "w3", "w_packed", "w_gate_packed"))
    H = oracle.noisy_logits(cpu["x"], cpu["w_gate"], cpu["w_noise"], None, cpu["eps"])[2]
    keep = oracle.batch_mask(H, m)
    G = oracle.masked_gates(H, keep)
    counts, offsets, perm, pos = oracle.masked_route(keep)
    imp = G.sum(axis=0)
    load = keep.sum(axis=0).astype(np.float64)
    ref = dict(H=H, keep=keep, gates=G, counts=counts, offsets=offsets, perm=perm, pos=pos,
               importance=imp, load=load, cv2_importance=oracle.cv_squared(imp),
               cv2_load=oracle.cv_squared(load))
    risky = _risky_experts(H, m, None)
    ok = ~keep[:, risky].any(axis=1)
    rng = np.random.default_rng(3)
    sample = np.sort(rng.choice(np.nonzero(ok)[0], size=96, replace=False))
    x = cpu["x"].double().numpy()
    y_ref = np.zeros((sample.size, cfg.d_model))
    for e in np.unique(np.nonzero(keep[sample])[1]):
        rows = np.nonzero(keep[sample, e])[0]
        ye = oracle.expert_relu(x[sample[rows]], inp["w1"][e].cpu(), inp["w2"][e].cpu())
        y_ref[rows] += G[sample[rows], e][:, None] * ye
    ref["y"] = None
    nr, nt, worst = check_mask_layer(cfg, out, ref, m, None, y_rows=sample, y_ref=y_ref)
    _say(f"[mask-full] flat256: ok risky experts={nr} excluded tokens={nt} worst_y={worst:.2e}")
