"""Host-side checks of the C ABI: the library loads, exports every function
include/moe.h declares, and rejects bad arguments before touching a GPU.
No call here reaches a kernel launch."""
import ctypes

import pytest

from sparsely_gated_mixture_noisy_amd import _lib as L
from sparsely_gated_mixture_noisy_amd.inputs import CONFIGS, MoEConfig

FAKE = 1 << 20  # a non-null, 256-byte aligned stand-in pointer (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_every_header_function(lib):
    names = L.header_functions()
    assert {"moe_gate", "moe_route", "moe_expert_ffn", "moe_combine", "moe_balance_loss",
            "moe_forward", "moe_workspace_size", "moe_status_string", "moe_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"ok"
    assert b"workspace" in lib.moe_status_string(L.MOE_ERR_WORKSPACE)
    assert lib.moe_status_string(99) == b"unknown status"


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_sizes(name):
    cfg = CONFIGS[name]
    n = L.workspace_size(cfg)
    assert n > 0 and n % 256 == 0
    # grows with the batch
    assert L.workspace_size(cfg, tokens=cfg.tokens * 2) > n


def _gate_call(lib, cfg, params=None, noise=None, ws_bytes=1 << 40, ws=FAKE, thr=None):
    c = L.make_config(cfg)
    p = params or L.moe_params(w_gate=FAKE, w_noise=FAKE, w1=FAKE, w2=FAKE, w3=FAKE,
                               w_gate_p=FAKE, w_noise_p=FAKE)
    n = noise or L.moe_noise(eps=FAKE, eps_p=FAKE)
    return lib.moe_gate(ctypes.byref(c), FAKE, ctypes.byref(p), ctypes.byref(n), FAKE, FAKE, thr,
                        ws, ws_bytes, None)


def test_invalid_configs_rejected_before_launch(lib):
    base = CONFIGS["flat256"]
    assert _gate_call(lib, base.replace(top_k=300)) == L.MOE_ERR_INVALID_ARG
    assert _gate_call(lib, base.replace(top_k=0)) == L.MOE_ERR_INVALID_ARG
    assert _gate_call(lib, base.replace(tokens=-1)) == L.MOE_ERR_INVALID_ARG
    assert _gate_call(lib, base.replace(d_model=100)) == L.MOE_ERR_UNSUPPORTED
    assert _gate_call(lib, base.replace(top_k=9)) == L.MOE_ERR_UNSUPPORTED
    assert _gate_call(lib, base.replace(n_experts=9000)) == L.MOE_ERR_UNSUPPORTED
    assert b"n_experts" in lib.moe_last_error()
    hier = CONFIGS["hier4096"]
    assert _gate_call(lib, hier.replace(k_groups=3)) == L.MOE_ERR_INVALID_ARG  # 3*2 != 4
    assert _gate_call(lib, hier.replace(n_groups=15)) == L.MOE_ERR_INVALID_ARG
    assert _gate_call(lib, hier, thr=FAKE) == L.MOE_ERR_INVALID_ARG


def test_missing_tensors_rejected(lib):
    cfg = CONFIGS["flat256"]
    no_noise = L.moe_params(w_gate=FAKE, w_noise=None, w1=FAKE, w2=FAKE)
    assert _gate_call(lib, cfg, params=no_noise) == L.MOE_ERR_INVALID_ARG
    assert _gate_call(lib, cfg, noise=L.moe_noise(eps=None, eps_p=None)) == L.MOE_ERR_INVALID_ARG
    c = L.make_config(CONFIGS["mixtral"])
    p = L.moe_params(w_gate=FAKE, w1=FAKE, w2=FAKE, w3=None)
    assert lib.moe_expert_ffn(ctypes.byref(c), FAKE, FAKE, FAKE, ctypes.byref(p), FAKE, FAKE,
                              1 << 40, None) == L.MOE_ERR_INVALID_ARG
    assert b"w3" in lib.moe_last_error()


def test_noisy_gate_without_noise_struct_rejected(lib):
    """A noisy layer called with noise == NULL is refused with a status, also
    for an empty batch (which reads no noise), instead of reading through
    the null pointer on the host."""
    for cfg in (CONFIGS["flat256"], CONFIGS["flat256"].replace(tokens=0),
                CONFIGS["hier4096"].replace(tokens=0)):
        c = L.make_config(cfg)
        p = L.moe_params(w_gate=FAKE, w_noise=FAKE, w_gate_p=FAKE, w_noise_p=FAKE)
        assert lib.moe_gate(ctypes.byref(c), FAKE, ctypes.byref(p), None, FAKE, FAKE, None,
                            FAKE, 1 << 40, None) == L.MOE_ERR_INVALID_ARG
        assert b"noise" in lib.moe_last_error()
        o = L.moe_outputs(y=FAKE, topk_idx=FAKE, topk_gate=FAKE, counts=FAKE)
        assert lib.moe_forward(ctypes.byref(c), FAKE, ctypes.byref(p), None, 1.0, 1.0,
                               ctypes.byref(o), FAKE, 1 << 40, None) == L.MOE_ERR_INVALID_ARG


def test_static_scratch_forward_refuses_layers_too_large(lib):
    """moe_forward_static takes layers whose workspace fits its 64 MiB static
    array (the 8192-token, 256-expert layer needs about 34 MiB) and refuses
    larger ones with MOE_ERR_WORKSPACE before touching a GPU."""
    assert L.workspace_size(CONFIGS["flat256"]) <= 64 << 20
    for cfg in (CONFIGS["mixtral"], CONFIGS["hier4096"], CONFIGS["flat256"].replace(tokens=20000)):
        assert L.workspace_size(cfg) > 64 << 20
        c = L.make_config(cfg)
        p = L.moe_params(w_gate=FAKE, w_noise=FAKE, w_gate_p=FAKE, w_noise_p=FAKE, w1=FAKE,
                         w2=FAKE, w3=FAKE)
        n = L.moe_noise(eps=FAKE, eps_p=FAKE)
        o = L.moe_outputs(y=FAKE)
        assert lib.moe_forward_static(ctypes.byref(c), FAKE, ctypes.byref(p), ctypes.byref(n),
                                      1.0, 1.0, ctypes.byref(o), None) == L.MOE_ERR_WORKSPACE
        assert b"static" in lib.moe_last_error()


def test_mask_requests_rejected_before_launch(lib):
    """moe_forward_mask refuses the hierarchy, a capacity (rows_per_expert sets
    the rows), rows_per_expert outside [1, tokens] and a missing workspace,
    before touching a GPU; its workspace size is 0 for such requests."""
    flat = CONFIGS["flat256"]
    assert L.mask_workspace_size(flat, 128) > 0
    p = L.moe_params(w_gate=FAKE, w_noise=FAKE, w_gate_p=FAKE, w_noise_p=FAKE, w1=FAKE, w2=FAKE)
    n = L.moe_noise(eps=FAKE, eps_p=FAKE)
    o = L.moe_mask_outputs(y=FAKE)
    for cfg, m, status in ((CONFIGS["hier4096"], 4, L.MOE_ERR_UNSUPPORTED),
                           (flat.replace(capacity=8), 8, L.MOE_ERR_INVALID_ARG),
                           (flat, 0, L.MOE_ERR_INVALID_ARG),
                           (flat, flat.tokens + 1, L.MOE_ERR_INVALID_ARG)):
        assert L.mask_workspace_size(cfg, m) == 0
        c = L.make_config(cfg)
        assert lib.moe_forward_mask(ctypes.byref(c), FAKE, ctypes.byref(p), ctypes.byref(n), m,
                                    None, 1.0, 1.0, ctypes.byref(o), FAKE, 1 << 40,
                                    None) == status
    c = L.make_config(flat)
    assert lib.moe_forward_mask(ctypes.byref(c), FAKE, ctypes.byref(p), ctypes.byref(n), 128, None,
                                1.0, 1.0, ctypes.byref(o), None, 0, None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_forward_mask(ctypes.byref(c), FAKE, ctypes.byref(p), ctypes.byref(n), 128, None,
                                1.0, 1.0, ctypes.byref(o), FAKE,
                                L.mask_workspace_size(flat, 128) - 1, None) == L.MOE_ERR_WORKSPACE


def test_workspace_checks(lib):
    cfg = CONFIGS["flat256"]
    need = L.workspace_size(cfg)
    assert _gate_call(lib, cfg, ws_bytes=need - 1) == L.MOE_ERR_WORKSPACE
    assert _gate_call(lib, cfg, ws=FAKE + 8) == L.MOE_ERR_WORKSPACE
    assert _gate_call(lib, cfg, ws=None) == L.MOE_ERR_WORKSPACE


def test_binding_raises_with_detail():
    cfg = CONFIGS["flat256"].replace(top_k=0)
    with pytest.raises(L.MoEError) as ei:
        L._check(_gate_call(L.load(), cfg), "moe_gate")
    assert ei.value.status == L.MOE_ERR_INVALID_ARG


def test_packed_table_sizes_and_rejections(lib):
    """Packed gate tables: one 32-expert block per started 32 experts of a
    group, both tables when noisy; none for fp32 gates."""
    assert L.packed_gate_size(CONFIGS["flat256"]) == 8 * 32 * 512 * 2 * 2
    assert L.packed_gate_size(CONFIGS["flat256"].replace(n_experts=40)) == 2 * 32 * 512 * 2 * 2
    assert L.packed_gate_size(CONFIGS["hier4096"]) == 16 * 8 * 32 * 512 * 2 * 2
    assert L.packed_gate_size(CONFIGS["mixtral"]) == 1 * 32 * 4096 * 1 * 2  # no noise table
    assert L.packed_gate_size(CONFIGS["tiny"]) == 0
    c = L.make_config(CONFIGS["tiny"])
    p = L.moe_params(w_gate=FAKE, w_noise=FAKE)
    assert lib.moe_pack_gate(ctypes.byref(c), ctypes.byref(p), FAKE, None) == L.MOE_ERR_UNSUPPORTED
    c = L.make_config(CONFIGS["flat256"])
    assert lib.moe_pack_gate(ctypes.byref(c), ctypes.byref(p), FAKE + 8, None) == \
        L.MOE_ERR_INVALID_ARG
    # an unaligned packed table is refused by the gate before any launch
    bad = L.moe_params(w_gate=FAKE, w_noise=FAKE, w_gate_packed=FAKE + 2)
    assert _gate_call(L.load(), CONFIGS["flat256"], params=bad) == L.MOE_ERR_INVALID_ARG
    bad = L.moe_params(w_gate=FAKE, w_noise=FAKE, w_gate_packed=FAKE)
    assert _gate_call(L.load(), CONFIGS["tiny"], params=bad) == L.MOE_ERR_UNSUPPORTED


def test_product_path_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No fallback: with the HIP library missing, the binding raises before
    any computation instead of computing the layer some other way."""
    from sparsely_gated_mixture_noisy_amd import _lib as L
    from sparsely_gated_mixture_noisy_amd.inputs import CONFIGS, make_inputs
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "libmoe.so"))
    monkeypatch.setattr(L, "_lib", None)
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg, seed=0)
    with pytest.raises(RuntimeError, match="missing"):
        L.forward(cfg, inp["x"], inp, inp)


def test_package_does_not_use_the_oracle():
    """The oracle is test infrastructure: nothing in the package imports it."""
    import os
    import re
    pkg = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "sparsely_gated_mixture_noisy_amd")
    pat = re.compile(r"^\s*(import|from)\s+oracle\b", re.M)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                with open(os.path.join(root, f)) as fh:
                    assert not pat.search(fh.read()), f
