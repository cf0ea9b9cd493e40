"""The sparse step in one launch (one token, bf16 rows, no next layer) against the
oracle: y_out = y + MLP_{S_M}(y) + MHA_{S_A}(y) (Deja Vu page, section 2.3, Eq. (1)
and (2)), element by element, on every shape class the launch plans differently
(full and partial column slices, one and many key splits, every head width, fp32
and bf16 caches, ReLU and GeLU), its edge cases (empty and full sets, counts below
and above capacity, indices outside the item range, in place), a workspace holding
garbage on entry, repeated calls, and the failure path of its in-launch waits
(forced from the host: every wait gives up, the kernel still ends, the output is
NaN and dv_check reports it)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from contextual_sparsity_mlp_amd import dv, synth
from contextual_sparsity_mlp_amd.synth import CONFIGS, LayerConfig
from gpu_helpers import TIGHT_ATTN, assert_close, banner, host
from oracle import dv_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"

SHAPES = {
    "c2": CONFIGS["c2"].with_(batch=1),
    "c3": CONFIGS["c3"].with_(batch=1),
    "c4": CONFIGS["c4"].with_(batch=1),
    # d = 264: one full 256-column slice and one of 8 columns; 37 keys: one split
    "d264": LayerConfig("d264", 21, d=264, F=1000, h=6, dh=64, batch=1, n_ctx=37, k_m=97,
                        k_a=2, r=24),
    # d = 64: a single partial slice; one key
    "d64": LayerConfig("d64", 22, d=64, F=256, h=2, dh=32, batch=1, n_ctx=1, k_m=16, k_a=1, r=8),
    "dh256": LayerConfig("dh256", 23, d=512, F=2048, h=3, dh=256, batch=1, n_ctx=300, k_m=205,
                         k_a=1, r=40),
    # 5000 keys: 40 key splits per head
    "long": LayerConfig("long", 24, d=128, F=512, h=4, dh=128, batch=1, n_ctx=5000, k_m=51,
                        k_a=3, r=16),
    "f32kv": LayerConfig("f32kv", 25, d=256, F=1024, h=4, dh=64, batch=1, n_ctx=130, k_m=100,
                         k_a=2, r=32, kvdtype="f32"),
}


@pytest.fixture(autouse=True)
def _one_launch():
    """Every test here runs the one-launch plan; the default plan is restored after."""
    dv.set_step_path(dv.PATH_ONE_LAUNCH)
    yield
    dv.set_step_path(dv.PATH_AUTO)


def i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def _layer(cfg, act="relu"):
    L = synth.make_layer(cfg, DEV, batch=1)
    layer = dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V, k_m=cfg.k_m, k_a=cfg.k_a,
                     scale=cfg.scale, act=dv.DV_ACT_GELU if act == "gelu" else dv.DV_ACT_RELU)
    return L, layer


def _oracle(cfg, L, y, S_M, S_A, act="relu"):
    ld = dict(W1t=host(L.W1t), W2t=host(L.W2t), Wq=host(L.Wq), Wo=host(L.Wo), K=host(L.K),
              V=host(L.V), act=act)
    ref, _ = O.decode_layer(host(y), ld, S_M, S_A, None, cfg.scale)
    return ref


def _run(cfg, layer, y, idx_m, cnt_m, cap_m, idx_a, cnt_a, cap_a, y_out=None, ws=None,
         garbage=None):
    if ws is None:
        ws = dv.workspace(dv.OP_DECODE_LAYER, batch=1, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                          n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=cap_m, max_count_a=cap_a)
    if garbage is not None:
        ws.fill_(garbage)
    if y_out is None:
        y_out = torch.full_like(y, np.nan)
    dv.decode_layer(layer, None, y, y_out, idx_m, cnt_m, cap_m, idx_a, cnt_a, cap_a,
                    None, None, None, None, ws)
    torch.cuda.synchronize()
    return y_out


def _sets(cfg, seed):
    S_M = synth.random_index_set(cfg.F, cfg.k_m, seed=seed).numpy()
    S_A = synth.random_index_set(cfg.h, cfg.k_a, seed=seed + 1).numpy()
    return S_M, S_A


@pytest.mark.parametrize("name", list(SHAPES))
def test_stream_parity(name):
    cfg = SHAPES[name]
    banner(f"one-launch sparse step {name}")
    L, layer = _layer(cfg)
    y = synth.make_y(cfg, DEV)
    S_M, S_A = _sets(cfg, cfg.cfg_id + 100)
    got = _run(cfg, layer, y, i32(S_M), i32([len(S_M)]), len(S_M), i32(S_A), i32([len(S_A)]),
               len(S_A), garbage=0xFF)
    ref = _oracle(cfg, L, y, S_M, S_A)
    assert_close(got.cpu().numpy(), ref, TIGHT_ATTN, f"stream {name}")
    # the same call again: bit-identical (fixed-order sums, whichever block took which item)
    got2 = _run(cfg, layer, y, i32(S_M), i32([len(S_M)]), len(S_M), i32(S_A), i32([len(S_A)]),
                len(S_A), garbage=0x00)
    assert torch.equal(got, got2), f"{name}: not deterministic"
    dv.check()


@pytest.mark.parametrize("name", ["d264", "c2"])
def test_stream_gelu(name):
    cfg = SHAPES[name]
    banner(f"one-launch sparse step gelu {name}")
    L, layer = _layer(cfg, act="gelu")
    y = synth.make_y(cfg, DEV)
    S_M, S_A = _sets(cfg, cfg.cfg_id + 200)
    got = _run(cfg, layer, y, i32(S_M), i32([len(S_M)]), len(S_M), i32(S_A), i32([len(S_A)]),
               len(S_A))
    assert_close(got.cpu().numpy(), _oracle(cfg, L, y, S_M, S_A, "gelu"), TIGHT_ATTN,
                 f"stream gelu {name}")


@pytest.mark.parametrize("name", ["d264", "d64", "f32kv", "c4"])
def test_stream_edges(name):
    cfg = SHAPES[name]
    banner(f"one-launch sparse step edges {name}")
    L, layer = _layer(cfg)
    y = synth.make_y(cfg, DEV)
    tol = TIGHT_ATTN
    E = np.zeros(0, dtype=np.int64)
    S_M, S_A = _sets(cfg, cfg.cfg_id + 300)

    def case(S_M, S_A, cap_m=None, cap_a=None, what=""):
        cap_m = len(S_M) if cap_m is None else cap_m
        cap_a = len(S_A) if cap_a is None else cap_a
        bm = torch.full((max(cap_m, 1),), -1, dtype=torch.int32, device=DEV)
        ba = torch.full((max(cap_a, 1),), -1, dtype=torch.int32, device=DEV)
        if len(S_M):
            bm[: len(S_M)] = i32(S_M)
        if len(S_A):
            ba[: len(S_A)] = i32(S_A)
        got = _run(cfg, layer, y, bm, i32([len(S_M)]), cap_m, ba, i32([len(S_A)]), cap_a)
        ref = _oracle(cfg, L, y, S_M, S_A)
        return assert_close(got.cpu().numpy(), ref, tol, f"{name} {what}")

    case(E, E, cap_m=5, cap_a=2, what="empty sets")
    case(E, E, cap_m=0, cap_a=0, what="no capacity")
    case(S_M, E, cap_a=0, what="no heads")
    case(E, S_A, cap_m=0, what="no neurons")
    case(np.arange(cfg.F), S_A, what="every neuron")
    case(S_M, np.arange(cfg.h), what="every head")
    case(S_M[: len(S_M) // 3], S_A[:1], cap_m=len(S_M), cap_a=len(S_A), what="count < cap")
    case(np.array([cfg.F - 1]), np.array([cfg.h - 1]), what="last neuron and head")
    # in place: y_out is y
    y2 = y.clone()
    _run(cfg, layer, y2, i32(S_M), i32([len(S_M)]), len(S_M), i32(S_A), i32([len(S_A)]),
         len(S_A), y_out=y2)
    assert_close(y2.cpu().numpy(), _oracle(cfg, L, y, S_M, S_A), tol, f"{name} in place")
    dv.check()


def test_stream_clamp_and_bad_indices():
    cfg = SHAPES["d264"]
    banner("one-launch sparse step clamp / bad indices")
    L, layer = _layer(cfg)
    y = synth.make_y(cfg, DEV)
    S_M = np.array([3, 10, cfg.F // 2, cfg.F - 1])
    S_A = np.array([1, 4])
    ref = _oracle(cfg, L, y, S_M, S_A)
    # device counts above the capacities: only the capacity's slots are read
    got = _run(cfg, layer, y, i32(S_M), i32([99]), 4, i32(S_A), i32([7]), 2)
    assert_close(got.cpu().numpy(), ref, TIGHT_ATTN, "clamped counts")
    # indices outside [0, F) and [0, h) contribute nothing
    bm = i32([3, -1, 10, cfg.F, cfg.F // 2, 1 << 30, cfg.F - 1])
    ba = i32([1, cfg.h, 4, -5])
    got = _run(cfg, layer, y, bm, i32([7]), 7, ba, i32([4]), 4)
    assert_close(got.cpu().numpy(), ref, TIGHT_ATTN, "bad indices skipped")
    dv.check()


def test_stream_many_calls_one_workspace():
    """Consecutive calls on one workspace and stream, on alternating layers and sets
    (each call's counters start from zero whatever the previous call left)."""
    cfg = SHAPES["dh256"]
    banner("one-launch sparse step, 12 calls on one workspace")
    cap_m, cap_a = cfg.k_m, cfg.k_a
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=1, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=cap_m, max_count_a=cap_a)
    cases = []
    for l in range(2):
        cl = cfg.with_(cfg_id=cfg.cfg_id + 10 * l)
        L, layer = _layer(cl)
        y = synth.make_y(cl, DEV)
        S_M, S_A = _sets(cl, 500 + l)
        cases.append((cl, L, layer, y, S_M, S_A, _oracle(cl, L, y, S_M, S_A)))
    outs = []
    for t in range(12):
        cl, L, layer, y, S_M, S_A, ref = cases[t % 2]
        y_out = torch.full_like(y, np.nan)
        dv.decode_layer(layer, None, y, y_out, i32(S_M), i32([len(S_M)]), cap_m, i32(S_A),
                        i32([len(S_A)]), cap_a, None, None, None, None, ws)
        outs.append((y_out, ref))
    torch.cuda.synchronize()
    for t, (y_out, ref) in enumerate(outs):
        assert_close(y_out.cpu().numpy(), ref, TIGHT_ATTN, f"call {t}")
    dv.check()


@pytest.mark.parametrize("name", ["d264", "c1"])
def test_wait_gives_up_loudly(name):
    """Every in-launch wait made to give up from the host (a target the producers never
    reach, a short poll limit): the launch still ends, every output element is NaN and
    dv_check reports DV_ETIMEOUT once; with the limits restored the same call is right.
    d264 runs the one-launch step, c1 (fp32 rows) the attention + waiting row-sum launch."""
    cfg = SHAPES.get(name) or CONFIGS[name]
    banner(f"in-launch wait failure path {name}")
    L, layer = _layer(cfg)
    y = synth.make_y(cfg, DEV)
    S_M, S_A = _sets(cfg, cfg.cfg_id + 400)
    args = (i32(S_M), i32([len(S_M)]), len(S_M), i32(S_A), i32([len(S_A)]), len(S_A))
    dv.check()                                   # nothing recorded before
    try:
        dv.debug_wait_limits(spins=64, extra=1)
        bad = _run(cfg, layer, y, *args)
    finally:
        dv.debug_wait_limits(0, 0)
    assert torch.isnan(bad).all(), f"{name}: outputs of a failed wait must be NaN"
    with pytest.raises(dv.DvError) as e:
        dv.check()
    assert e.value.code == dv.DV_ETIMEOUT
    dv.check()                                   # the record was cleared
    good = _run(cfg, layer, y, *args)
    tol = 1e-5 if cfg.wdtype == "f32" else TIGHT_ATTN
    assert_close(good.cpu().numpy(), _oracle(cfg, L, y, S_M, S_A), tol, f"{name} restored")
    dv.check()
