"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases run the whole layer through the oracle; the five full-size
workloads compare routing and gates over every token, layer outputs on a
sample of tokens, and the balance statistics."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_check import (check_balance, check_close, check_gate, check_routing, excluded, np_,
                       sampled_outputs, top_k1_sets)
from sparsely_gated_mixture_noisy_amd import _lib as L
from sparsely_gated_mixture_noisy_amd.inputs import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

RTOL = {"bf16": 2e-2, "f32": 1e-4}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def cpu_inputs(inp):
    return {k: (v.detach().to("cpu") if v is not None else None) for k, v in inp.items()}


def run_staged(cfg, inp):
    """gate -> route -> experts -> combine -> balance, one entry point each."""
    x = inp["x"]
    ws = L.workspace(cfg, x.shape[0])
    idx, gate, thr = L.gate(cfg, x, inp, inp, ws=ws)
    counts, offsets, perm, inv, _ = L.route(cfg, idx, ws=ws)
    ys = L.expert_ffn(cfg, x, perm, offsets, inp, ws=ws)
    y = L.combine(cfg, ys, inv, gate)
    imp, load, out = L.balance_loss(cfg, x, inp, idx, gate, thr, perm, offsets, 1.0, 1.0, ws=ws)
    torch.cuda.synchronize()
    return dict(idx=idx, gate=gate, thr=thr, counts=counts, offsets=offsets, perm=perm, inv=inv,
                y_sorted=ys, y=y, importance=imp, load=load, balance=out)


SMALL = {
    "tiny": CONFIGS["tiny"],
    "tiny_ragged": CONFIGS["tiny"].replace(tokens=77),
    "tiny_k_eq_E": CONFIGS["tiny"].replace(tokens=100, top_k=8),
    "tiny_swiglu": CONFIGS["tiny"].replace(tokens=90, ffn="swiglu", noisy=False),
    "tiny_hier": CONFIGS["tiny"].replace(tokens=123, n_experts=12, n_groups=3, k_groups=2,
                                         k_per_group=2, top_k=4, gate_std=0.3),
    "flat256_t1000": CONFIGS["flat256"].replace(tokens=1000),
    "flat256_k1": CONFIGS["flat256"].replace(tokens=333, top_k=1),
    "zipf2048_t2000": CONFIGS["zipf2048"].replace(tokens=2000),
    "hier4096_t300": CONFIGS["hier4096"].replace(tokens=300),
    "hier_g16_e64": CONFIGS["hier4096"].replace(tokens=700, n_experts=1024),
    "swiglu_bf16_small": CONFIGS["mixtral"].replace(tokens=200, d_model=512, d_hidden=1536),
    # fused expert kernel with 2 and 8 hidden chunks of 256 units
    "fused_h512": CONFIGS["flat256"].replace(tokens=600, d_hidden=512),
    "fused_h2048": CONFIGS["flat256"].replace(tokens=400, d_hidden=2048),
    # gate input tile in LDS at its largest d_model, and read from global above it
    "gate_d1024": CONFIGS["flat256"].replace(tokens=300, d_model=1024, n_experts=64),
    "gate_d1088": CONFIGS["flat256"].replace(tokens=300, d_model=1088, n_experts=40, top_k=3),
    # the largest expert count and top-k the library takes
    "e8192_k8": CONFIGS["flat256"].replace(tokens=200, d_model=64, d_hidden=128, n_experts=8192,
                                           top_k=8),
    "flat_k8": CONFIGS["flat256"].replace(tokens=300, top_k=8),
    "flat_noise_free": CONFIGS["flat256"].replace(tokens=300, noisy=False),
    # the large-tile grouped GEMMs (>= 256 rows per expert on average), ragged tiles
    "big_swiglu": CONFIGS["mixtral"].replace(tokens=1200, d_model=512, d_hidden=1536, n_experts=4),
    "big_relu_d256": CONFIGS["flat256"].replace(tokens=1500, d_model=256, d_hidden=512,
                                                n_experts=8, top_k=2),
    # the 256-wide column tiles of the big GEMMs with a ragged last column tile
    "big_relu_d320": CONFIGS["flat256"].replace(tokens=1300, d_model=320, d_hidden=640,
                                                n_experts=4, top_k=1),
    # 32 column tiles in the first GEMM: the XCD-grouped tile order of the
    # big GEMMs (the second GEMM, 2 column tiles, keeps the plain order)
    "big_swiglu_ncol32": CONFIGS["mixtral"].replace(tokens=1100, d_model=512, d_hidden=4096,
                                                    n_experts=4),
    "big_relu_ncol32": CONFIGS["flat256"].replace(tokens=1100, d_model=512, d_hidden=8192,
                                                  n_experts=4, top_k=1),
    # one group, then one expert: the hierarchy at k = 1
    "hier_k1": CONFIGS["hier4096"].replace(tokens=257, n_experts=160, k_groups=1,
                                           k_per_group=1, top_k=1),
    # experts in four gate blocks, the last one partial
    "flat_e1000": CONFIGS["zipf2048"].replace(tokens=400, n_experts=1000, bias="none"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_layer(name):
    cfg = SMALL[name]
    _say(f"[parity] {name}: {cfg}")
    inp = make_inputs(cfg, seed=0, device="cuda")
    got = run_staged(cfg, inp)
    ref = oracle.forward(cpu_inputs(inp), cfg)
    excl = excluded(ref)
    rep = {}
    check_gate(got["idx"], got["gate"], ref, excl, thr=got["thr"], report=rep)
    check_routing(got["counts"], got["offsets"], got["perm"], got["inv"], got["idx"], ref, excl,
                  cfg.top_k)
    rows = np.nonzero(~excl)[0]
    worst = check_close(got["y"], ref["y"], RTOL[cfg.dtype], rows=rows)
    check_balance(got["importance"], got["load"], got["balance"], ref, excl, ref["idx"],
                  k1_sets=top_k1_sets(ref, cfg), smooth=(cfg.noisy and not cfg.hierarchical))
    # moe_forward gives bitwise the staged results
    fo = L.forward(cfg, inp["x"], inp, inp)
    torch.cuda.synchronize()
    for a, b in [(fo.y, got["y"]), (fo.topk_idx, got["idx"]), (fo.topk_gate, got["gate"]),
                 (fo.counts, got["counts"]), (fo.importance, got["importance"]),
                 (fo.load, got["load"]), (fo.balance, got["balance"])]:
        assert torch.equal(a, b)
    _say(f"[parity] {name}: ok excluded={rep['excluded']} worst_y={worst:.2e}")


@pytest.mark.parametrize("name", list(CONFIGS))
def test_full_size(name):
    """Each workload at its full size, twice: through the staged entry points
    on the plain tables, and through moe_forward on the packed expert and
    gate tables, the launch configuration the benchmark times.  Both are
    compared with the oracle: gates and routing over every token, the
    balance statistics, and y on sampled included tokens."""
    cfg = CONFIGS[name]
    _say(f"[parity-full] {name}: {cfg}")
    inp = make_inputs(cfg, seed=0, device="cuda")
    got = run_staged(cfg, inp)
    binp = L.packed_params(cfg, inp)
    fo = L.forward(cfg, inp["x"], binp, binp, save=True)
    torch.cuda.synchronize()
    bench = dict(idx=fo.topk_idx, gate=fo.topk_gate, thr=fo.thr, counts=fo.counts,
                 offsets=fo.offsets, perm=fo.perm, inv=fo.inv, y=fo.y, importance=fo.importance,
                 load=fo.load, balance=fo.balance)
    cin = cpu_inputs({k: v for k, v in inp.items() if k not in ("w1", "w2", "w3")})
    ref = oracle.forward(cin, cfg, with_experts=False)
    excl = excluded(ref)
    rng = np.random.default_rng(1)
    inc = np.nonzero(~excl)[0]
    sample = np.sort(rng.choice(inc, size=min(96, inc.size), replace=False))
    y_ref = sampled_outputs(cfg, inp, cin["x"], ref, sample)
    for label, res in (("staged, plain tables", got), ("moe_forward, packed tables", bench)):
        _say(f"[parity-full] {name}: {label}")
        rep = {}
        check_gate(res["idx"], res["gate"], ref, excl, thr=res["thr"], report=rep)
        check_routing(res["counts"], res["offsets"], res["perm"], res["inv"], res["idx"], ref,
                      excl, cfg.top_k)
        check_balance(res["importance"], res["load"], res["balance"], ref, excl, ref["idx"],
                      k1_sets=top_k1_sets(ref, cfg),
                      smooth=(cfg.noisy and not cfg.hierarchical))
        worst = check_close(res["y"][torch.from_numpy(sample).cuda()], y_ref, RTOL[cfg.dtype])
        _say(f"[parity-full] {name}: {label} ok excluded={rep['excluded']} worst_y={worst:.2e}")
    # the packed tables hold the same values in another order: same bits
    assert torch.equal(fo.y, got["y"]) and torch.equal(fo.topk_idx, got["idx"])
    assert torch.equal(fo.topk_gate, got["gate"]) and torch.equal(fo.balance, got["balance"])
    c = np_(got["counts"])
    _say(f"[parity-full] {name}: counts max/mean={c.max() / max(c.mean(), 1e-9):.1f} "
         f"zero={int((c == 0).sum())}")


def test_determinism_bitwise():
    cfg = CONFIGS["flat256"]
    inp = make_inputs(cfg, seed=3, device="cuda")
    f = L.Forward(cfg, inp["x"], inp, inp)
    a = f()
    y1 = a.y.clone(); b1 = a.balance.clone(); g1 = a.topk_gate.clone()
    for _ in range(3):
        b = f()
        torch.cuda.synchronize()
        assert torch.equal(b.y, y1) and torch.equal(b.balance, b1) and torch.equal(b.topk_gate, g1)


def test_empty_batch():
    cfg = CONFIGS["flat256"].replace(tokens=0)
    inp = make_inputs(cfg, seed=0, device="cuda")
    fo = L.forward(cfg, inp["x"], inp, inp)
    torch.cuda.synchronize()
    assert fo.y.shape == (0, cfg.d_model)
    assert int(fo.counts.sum()) == 0
    assert fo.balance.tolist() == [0.0, 0.0, 0.0]


def test_single_token_and_single_expert():
    for cfg in (CONFIGS["flat256"].replace(tokens=1),
                CONFIGS["flat256"].replace(tokens=50, n_experts=1, top_k=1),
                CONFIGS["tiny"].replace(tokens=5, n_experts=1, top_k=1)):
        inp = make_inputs(cfg, seed=0, device="cuda")
        got = run_staged(cfg, inp)
        ref = oracle.forward(cpu_inputs(inp), cfg)
        excl = excluded(ref)
        check_gate(got["idx"], got["gate"], ref, excl)
        check_close(got["y"], ref["y"], RTOL[cfg.dtype], rows=np.nonzero(~excl)[0])


def test_identical_tokens_max_skew():
    """Every token the same and no noise: all T rows go to the same k experts
    (ties in the bf16 scores fall to the lower index, as in the oracle)."""
    cfg = CONFIGS["flat256"].replace(tokens=2048, noisy=False)
    inp = make_inputs(cfg, seed=0, device="cuda")
    inp["x"] = inp["x"][:1].expand(cfg.tokens, -1).contiguous()
    got = run_staged(cfg, inp)
    ref = oracle.forward(cpu_inputs(inp), cfg)
    excl = excluded(ref)
    assert not excl.any()
    c = np_(got["counts"])
    assert (np.sort(c)[-cfg.top_k:] == cfg.tokens).all() and c.sum() == cfg.tokens * cfg.top_k
    check_gate(got["idx"], got["gate"], ref, excl)
    check_routing(got["counts"], got["offsets"], got["perm"], got["inv"], got["idx"], ref, excl,
                  cfg.top_k)
    check_close(got["y"], ref["y"], RTOL[cfg.dtype])


def test_half_experts_starved_by_bias():
    """A bias of -1e4 on the odd experts: they receive no rows at all."""
    cfg = CONFIGS["flat256"].replace(tokens=1500)
    inp = make_inputs(cfg, seed=0, device="cuda")
    b = torch.zeros(cfg.n_experts, dtype=torch.float32, device="cuda")
    b[1::2] = -1e4
    inp["bias"] = b
    got = run_staged(cfg, inp)
    ref = oracle.forward(cpu_inputs(inp), cfg)
    excl = excluded(ref)
    c = np_(got["counts"])
    assert (c[1::2] == 0).all()
    check_gate(got["idx"], got["gate"], ref, excl, thr=got["thr"])
    check_routing(got["counts"], got["offsets"], got["perm"], got["inv"], got["idx"], ref, excl,
                  cfg.top_k)
    check_close(got["y"], ref["y"], RTOL[cfg.dtype], rows=np.nonzero(~excl)[0])
    check_balance(got["importance"], got["load"], got["balance"], ref, excl, ref["idx"],
                  k1_sets=top_k1_sets(ref, cfg))


def test_route_x_sorted_gather():
    cfg = CONFIGS["flat256"].replace(tokens=700)
    inp = make_inputs(cfg, seed=0, device="cuda")
    idx, gate, _ = L.gate(cfg, inp["x"], inp, inp)
    counts, offsets, perm, inv, xs = L.route(cfg, idx, x=inp["x"])
    torch.cuda.synchronize()
    assert torch.equal(xs, inp["x"][(perm // cfg.top_k).long()])
    # experts on the gathered rows give bitwise the gathered-in-kernel result
    y1 = L.expert_ffn(cfg, inp["x"], perm, offsets, inp)
    y2 = L.expert_ffn(cfg, xs, None, offsets, inp, tokens=cfg.tokens)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("tokens", [1000, 8192])
def test_packed_experts_match_unpacked_bitwise(tokens):
    """The repacked expert tables hold the same values in stream order: the
    expert stage gives bitwise the result of the unpacked tables, and the
    whole layer stays within the oracle's tolerance."""
    cfg = CONFIGS["flat256"].replace(tokens=tokens)
    inp = make_inputs(cfg, seed=5, device="cuda")
    packed = L.pack_experts(cfg, inp)
    assert packed is not None and packed.numel() * 2 == L.packed_experts_size(cfg)
    idx, gate, _ = L.gate(cfg, inp["x"], inp, inp)
    counts, offsets, perm, inv, _ = L.route(cfg, idx)
    y_plain = L.expert_ffn(cfg, inp["x"], perm, offsets, inp)
    only_packed = {"w_packed": packed}
    y_packed = L.expert_ffn(cfg, inp["x"], perm, offsets, only_packed)
    torch.cuda.synchronize()
    assert torch.equal(y_plain, y_packed)
    fo = L.forward(cfg, inp["x"], dict(inp, w_packed=packed), inp)
    torch.cuda.synchronize()
    assert torch.equal(fo.y, L.combine(cfg, y_plain, inv, gate))


def test_pack_rejects_unsupported_layers():
    for cfg in (CONFIGS["tiny"], CONFIGS["mixtral"].replace(tokens=4, n_experts=2, d_hidden=256)):
        assert L.packed_experts_size(cfg) == 0
        inp = make_inputs(cfg.replace(tokens=4), seed=0, device="cuda")
        assert L.pack_experts(cfg, inp) is None


PACK_GATE_CASES = {
    "flat256_t1000": CONFIGS["flat256"].replace(tokens=1000),
    "flat_e40": CONFIGS["flat256"].replace(tokens=500, n_experts=40, top_k=3),
    "zipf2048_t2000": CONFIGS["zipf2048"].replace(tokens=2000),
    "hier_eg40": CONFIGS["hier4096"].replace(tokens=300, n_experts=16 * 40),
    "mixtral_t64": CONFIGS["mixtral"].replace(tokens=64),
}


@pytest.mark.parametrize("name", list(PACK_GATE_CASES))
def test_packed_gate_matches_unpacked_bitwise(name):
    """The repacked gate tables hold the same values in the order the gate
    kernels stream them: gate, smooth-load and whole-layer results are
    bitwise those of the unpacked tables (expert counts that are not a
    multiple of 32 exercise the padded last block)."""
    cfg = PACK_GATE_CASES[name]
    _say(f"[packed gate] {name}: {cfg}")
    inp = make_inputs(cfg, seed=11, device="cuda")
    gp = L.pack_gate(cfg, inp)
    assert gp is not None and gp.numel() * 2 == L.packed_gate_size(cfg)
    packed = dict(inp, w_gate_packed=gp)
    a = L.gate(cfg, inp["x"], inp, inp)
    b = L.gate(cfg, inp["x"], packed, inp)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert (u is None and v is None) or torch.equal(u, v)
    fa = L.forward(cfg, inp["x"], inp, inp)
    fb = L.forward(cfg, inp["x"], packed, inp)
    torch.cuda.synchronize()
    for key in ("y", "topk_idx", "topk_gate", "counts", "importance", "load", "balance"):
        assert torch.equal(getattr(fa, key), getattr(fb, key)), key


@pytest.mark.parametrize("base", ["flat256", "hier4096", "zipf2048"])
def test_nan_row_keeps_real_experts(base):
    """A token whose input row is NaN scores NaN everywhere; its selection
    ranks NaN as -inf, so it still keeps k experts inside [0, E) (the lowest
    indices, as among equal scores) and the routing, the experts and the
    combine stay in bounds; every other token matches the oracle."""
    cfg = CONFIGS[base].replace(tokens=300)
    inp = make_inputs(cfg, seed=0, device="cuda")
    bad = 77
    inp["x"][bad] = float("nan")
    fo = L.forward(cfg, inp["x"], inp, inp, save=True)
    torch.cuda.synchronize()
    idx = np_(fo.topk_idx)
    assert ((idx >= 0) & (idx < cfg.n_experts)).all()
    c = np_(fo.counts)
    assert int(c.sum()) == cfg.tokens * cfg.top_k
    perm, inv = np_(fo.perm), np_(fo.inv)
    assert (np.sort(perm) == np.arange(perm.size)).all() and (perm[inv] == np.arange(perm.size)).all()
    if not cfg.hierarchical:
        assert (idx[bad] == np.arange(cfg.top_k)).all()
    ref = oracle.forward(cpu_inputs(inp), cfg)
    excl = excluded(ref)
    excl[bad] = True
    check_gate(fo.topk_idx, fo.topk_gate, ref, excl)
    check_close(fo.y, ref["y"], RTOL[cfg.dtype], rows=np.nonzero(~excl)[0])


def test_route_drops_expert_ids_outside_the_layer():
    """moe_route on caller-supplied indices, some of them outside [0, E)
    (-1, E, the largest int32): those assignments take no row (inv = -1),
    and the others are grouped exactly as the stable routing of the valid
    assignments alone."""
    cfg = CONFIGS["flat256"].replace(tokens=500, n_experts=40, top_k=3)
    rng = np.random.default_rng(5)
    idx = np.stack([np.sort(rng.choice(cfg.n_experts, size=3, replace=False))
                    for _ in range(cfg.tokens)]).astype(np.int32)
    bad = rng.choice(idx.size, size=37, replace=False)
    idx.reshape(-1)[bad] = rng.choice([-1, cfg.n_experts, 2 ** 31 - 1], size=bad.size)
    counts, offsets, perm, inv, _ = L.route(cfg, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < cfg.n_experts)
    want_counts = np.bincount(flat[valid], minlength=cfg.n_experts)
    assert (np_(counts) == want_counts).all()
    assert (np_(offsets) == np.concatenate([[0], np.cumsum(want_counts)])).all()
    a = np.nonzero(valid)[0]
    order = a[np.argsort(flat[a], kind="stable")]   # by expert, assignments ascending
    n = order.size
    assert (np_(perm)[:n] == order).all() and (np_(perm)[n:] == 0).all()
    want_inv = np.full(flat.size, -1)
    want_inv[order] = np.arange(n)
    assert (np_(inv) == want_inv).all()
