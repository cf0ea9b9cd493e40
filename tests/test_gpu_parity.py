"""HIP path vs the CPU oracle, element by element, through the C ABI.

Every case uses seeded synthetic inputs from contextual_sparsity_mlp_amd.synth; the
oracle receives host copies of exactly the tensors the GPU reads.  Index sets are
compared bit-exactly when both sides select from the same fp32 scores, and with
certified rounding swaps only when each side computed its own scores.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from contextual_sparsity_mlp_amd import dv, synth
from contextual_sparsity_mlp_amd.synth import CONFIGS, LayerConfig
from gpu_helpers import (BOUND_BF16, BOUND_F32, TIGHT_ATTN, TIGHT_MLP, assert_close, banner,
                         check_sets_certified, host, score_bound)
from oracle import dv_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    dv.lib()
    yield
    torch.cuda.synchronize()


# Ragged shapes: d not a multiple of the 512-element wave-load, F and h not powers of
# two, short and long caches, odd batch, every head width the kernels take.
RAGGED = {
    "c1": CONFIGS["c1"],
    "bf16-ragged": LayerConfig("bf16-ragged", 11, d=264, F=1000, h=6, dh=64, batch=3, n_ctx=37,
                               k_m=97, k_a=2, r=24, union=True),
    "f32-ragged": LayerConfig("f32-ragged", 12, d=72, F=300, h=5, dh=32, batch=2, n_ctx=5,
                              k_m=31, k_a=3, r=7, wdtype="f32", kvdtype="f32", union=True),
    "bf16-dh256": LayerConfig("bf16-dh256", 13, d=512, F=2048, h=3, dh=256, batch=1, n_ctx=300,
                              k_m=205, k_a=1, r=40),
    "long-ctx": LayerConfig("long-ctx", 14, d=128, F=512, h=4, dh=128, batch=2, n_ctx=5000,
                            k_m=51, k_a=3, r=16, union=True),
    "mixed-kv": LayerConfig("mixed-kv", 15, d=256, F=1024, h=4, dh=64, batch=5, n_ctx=130,
                            k_m=100, k_a=2, r=32, kvdtype="f32", union=True),
    "n1": LayerConfig("n1", 16, d=64, F=256, h=2, dh=32, batch=1, n_ctx=1, k_m=16, k_a=1, r=8),
    # batches on the matrix-core row dots: a second, partial token tile (17) and a
    # third token group (35)
    "b17": LayerConfig("b17", 17, d=384, F=700, h=5, dh=32, batch=17, n_ctx=40, k_m=77, k_a=2,
                       r=20, union=True),
    "b35": LayerConfig("b35", 18, d=256, F=520, h=3, dh=64, batch=35, n_ctx=9, k_m=30, k_a=1,
                       r=12, union=True),
}
SMALL = list(RAGGED)
FULL = ["c2", "c3"]


def cfg_of(name):
    return RAGGED[name] if name in RAGGED else CONFIGS[name]


def tol_of(cfg, tight):
    return BOUND_F32 if cfg.wdtype == "f32" else min(BOUND_BF16, tight)


def i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=DEV)


def put_set(S, cap):
    """Device index list of capacity `cap` holding ascending S, and its device count."""
    buf = torch.full((max(cap, 1),), -1, dtype=torch.int32, device=DEV)
    if len(S):
        buf[: len(S)] = i32(S)
    return buf, i32([len(S)])


# --------------------------------------------------------------------------- #
# A1 predictor                                                                #
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("name", SMALL + FULL)
def test_predict_parity(name):
    cfg = cfg_of(name)
    banner(f"predict {name}")
    P = synth.make_predictor(cfg, DEV)
    y = synth.make_y(cfg, DEV)
    for A, Bm in ((P["A_M"], P["B_M"]), (P["A_A"], P["B_A"])):
        N = Bm.shape[1]
        s = torch.empty((cfg.batch, N), dtype=torch.float32, device=DEV)
        ws = dv.workspace(dv.OP_PREDICT, batch=cfg.batch, d=cfg.d, r=cfg.r, N=N)
        dv.predict(y, A, Bm, s, ws)
        ref = O.predict_scores(host(y), host(A), host(Bm))
        got = s.cpu().numpy()
        bound = score_bound(host(y), host(A), host(Bm))
        assert np.all(np.abs(got - ref) <= bound), f"{name}: score outside the certified bound"
        assert_close(got, ref, tol_of(cfg, TIGHT_MLP), f"{name} scores N={N}")
        s2 = torch.empty_like(s)
        dv.predict(y, A, Bm, s2, ws)
        assert torch.equal(s, s2), "predict not deterministic"


@pytest.mark.parametrize("batch", [1, 16])
def test_predict_c4(batch):
    """The OPT-175B-shaped predictor (d = 12288, r = 1000, 49152 neurons and 96 heads):
    one token on the wave path, 16 on the matrix cores; every score inside its
    certified bound and close to the oracle's."""
    cfg = CONFIGS["c4"]
    banner(f"predict c4 batch={batch}")
    P = synth.make_predictor(cfg, DEV)
    y = synth.make_y(cfg, DEV, batch=batch)
    yh = host(y)
    for A, Bm in ((P["A_M"], P["B_M"]), (P["A_A"], P["B_A"])):
        N = Bm.shape[1]
        s = torch.empty((batch, N), dtype=torch.float32, device=DEV)
        ws = dv.workspace(dv.OP_PREDICT, batch=batch, d=cfg.d, r=cfg.r, N=N)
        dv.predict(y, A, Bm, s, ws)
        Ah, Bh = host(A), host(Bm)
        ref = O.predict_scores(yh, Ah, Bh)
        got = s.cpu().numpy()
        bound = score_bound(yh, Ah, Bh)
        assert np.all(np.abs(got - ref) <= bound), f"c4 B={batch} N={N}: score outside the bound"
        assert_close(got, ref, TIGHT_MLP, f"c4 B={batch} scores N={N}")


# --------------------------------------------------------------------------- #
# A2 top-k / union: bit-exact on identical scores                             #
# --------------------------------------------------------------------------- #

def _topk_case(scores_np, k, union):
    B, N = scores_np.shape
    s = torch.as_tensor(scores_np.astype(np.float32), device=DEV)
    cap = min(N, B * k) if union else B * k
    idx = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    ws = dv.workspace(dv.OP_SELECT_TOPK, batch=B, N=N)
    dv.select_topk(s, k, union, idx, cnt, ws)
    ref = O.select_sets(scores_np.astype(np.float32).astype(np.float64), k, union)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    if union:
        assert cnt[0] == len(ref), f"union count {cnt[0]} != {len(ref)}"
        assert np.array_equal(idx[: cnt[0]], ref), "union set differs"
    else:
        for b in range(B):
            assert cnt[b] == k
            assert np.array_equal(idx[b * k:(b + 1) * k], ref[b]), f"row {b} differs"


TOPK_CASES = [
    # (B, N, k, union, kind)
    (1, 49152, 4915, 1, "normal"), (1, 96, 19, 1, "normal"), (4, 28672, 3441, 1, "normal"),
    (16, 49152, 4915, 1, "normal"), (3, 1000, 97, 0, "normal"), (2, 37, 0, 1, "normal"),
    (2, 37, 37, 1, "normal"), (2, 37, 37, 0, "normal"), (1, 1, 1, 1, "normal"),
    (5, 4099, 400, 1, "ties"), (3, 5000, 1234, 0, "ties"), (1, 8192, 100, 1, "const"),
    (2, 300, 31, 1, "zeros"), (7, 96, 19, 1, "ties"), (1, 12289, 6000, 1, "ties"),
    (3, 64, 5, 1, "huge"),
]


@pytest.mark.parametrize("B,N,k,union,kind", TOPK_CASES)
def test_select_topk_bitexact(B, N, k, union, kind):
    banner(f"select_topk B={B} N={N} k={k} union={union} {kind}")
    rng = np.random.default_rng(1000 + B * 7 + N + k)
    if kind == "normal":
        s = rng.standard_normal((B, N))
    elif kind == "ties":
        s = np.round(rng.standard_normal((B, N)) * 4) / 4          # heavy ties
    elif kind == "const":
        s = np.full((B, N), 0.75)
    elif kind == "zeros":
        s = rng.choice([-0.0, 0.0, -1.0, 1.0], size=(B, N))
    else:
        s = rng.standard_normal((B, N)) * 1e30
        s[:, ::7] = -3e38
    _topk_case(s, k, bool(union))


def test_select_topk_gpu_scores():
    """Top-k of the GPU's own c4 predictor scores equals the oracle's top-k of them."""
    cfg = CONFIGS["c4"]
    banner("select_topk on c4 predictor scores")
    P = synth.make_predictor(cfg, DEV)
    y = synth.make_y(cfg, DEV, batch=4)
    s = torch.empty((4, cfg.F), dtype=torch.float32, device=DEV)
    dv.predict(y, P["A_M"], P["B_M"], s, dv.workspace(dv.OP_PREDICT, batch=4, d=cfg.d, r=cfg.r,
                                                       N=cfg.F))
    _topk_case(s.cpu().numpy().astype(np.float64), cfg.k_m, True)
    _topk_case(s.cpu().numpy().astype(np.float64), cfg.k_m, False)


# --------------------------------------------------------------------------- #
# A3 sparse MLP                                                               #
# --------------------------------------------------------------------------- #

def _mlp_case(cfg, L, y, S, accumulate=False, cap=None, act="relu"):
    B = y.shape[0]
    cap = len(S) if cap is None else cap
    idx, cnt = put_set(S, cap)
    code = dv.DV_ACT_GELU if act == "gelu" else dv.DV_ACT_RELU
    out = torch.full((B, cfg.d), 0.5 if accumulate else np.nan, dtype=torch.float32, device=DEV)
    ws = dv.workspace(dv.OP_SPARSE_MLP, batch=B, d=cfg.d, max_count_m=cap)
    dv.sparse_mlp(y, L.W1t, L.W2t, idx, cnt, cap, out, accumulate, ws, act=code)
    ref = O.sparse_mlp(host(y), host(L.W1t), host(L.W2t), S, act) + (0.5 if accumulate else 0.0)
    got = out.cpu().numpy()
    out2 = torch.full_like(out, 0.5 if accumulate else np.nan)
    dv.sparse_mlp(y, L.W1t, L.W2t, idx, cnt, cap, out2, accumulate, ws, act=code)
    assert torch.equal(out, out2), "sparse_mlp not deterministic"
    return got, ref


@pytest.mark.parametrize("name", SMALL + FULL)
def test_sparse_mlp_parity(name):
    cfg = cfg_of(name)
    banner(f"sparse_mlp {name}")
    L = synth.make_layer(cfg, DEV, with_kv=False)
    y = synth.make_y(cfg, DEV)
    S = synth.random_index_set(cfg.F, cfg.k_m, seed=cfg.cfg_id).numpy()
    got, ref = _mlp_case(cfg, L, y, S)
    assert_close(got, ref, tol_of(cfg, TIGHT_MLP), f"mlp {name}")


@pytest.mark.parametrize("name", ["c1", "bf16-ragged", "f32-ragged", "c2"])
def test_sparse_mlp_gelu(name):
    """sigma = GeLU (the page's other named activation)."""
    cfg = cfg_of(name)
    banner(f"sparse_mlp gelu {name}")
    L = synth.make_layer(cfg, DEV, with_kv=False)
    y = synth.make_y(cfg, DEV)
    S = synth.random_index_set(cfg.F, cfg.k_m, seed=cfg.cfg_id + 40).numpy()
    got, ref = _mlp_case(cfg, L, y, S, act="gelu")
    assert_close(got, ref, tol_of(cfg, TIGHT_MLP), f"gelu mlp {name}")
    got_a, ref_a = _mlp_case(cfg, L, y, S, accumulate=True, act="gelu")
    assert_close(got_a, ref_a, tol_of(cfg, TIGHT_MLP), f"gelu mlp accumulate {name}")


# mixed-kv (batch 5, d 256) and b17 take the matrix-core row dots and row sums
@pytest.mark.parametrize("name", ["c1", "bf16-ragged", "f32-ragged", "mixed-kv", "b17"])
def test_sparse_mlp_edges(name):
    cfg = cfg_of(name)
    banner(f"sparse_mlp edges {name}")
    L = synth.make_layer(cfg, DEV, with_kv=False)
    y = synth.make_y(cfg, DEV)
    tol = tol_of(cfg, TIGHT_MLP)
    # empty set: exactly zero (and exactly the old value with accumulate)
    got, _ = _mlp_case(cfg, L, y, np.zeros(0, dtype=np.int64), cap=5)
    assert np.array_equal(got, np.zeros_like(got)), "empty set must give exact zero"
    got, _ = _mlp_case(cfg, L, y, np.zeros(0, dtype=np.int64), accumulate=True, cap=3)
    assert np.array_equal(got, np.full_like(got, 0.5))
    # every neuron: the dense MLP
    got, ref = _mlp_case(cfg, L, y, np.arange(cfg.F))
    assert_close(got, ref, tol, "mlp S=all")
    # accumulate
    S = synth.random_index_set(cfg.F, 7, seed=3).numpy()
    got, ref = _mlp_case(cfg, L, y, S, accumulate=True)
    assert_close(got, ref, tol, "mlp accumulate")
    # count below capacity; a single neuron; the last neuron
    got, ref = _mlp_case(cfg, L, y, S[:4], cap=50)
    assert_close(got, ref, tol, "mlp count < cap")
    got, ref = _mlp_case(cfg, L, y, np.array([cfg.F - 1]))
    assert_close(got, ref, tol, "mlp last neuron")


@pytest.mark.parametrize("name", ["bf16-ragged", "mixed-kv", "b17"])
def test_sparse_mlp_device_count_clamped_and_bad_indices(name):
    cfg = RAGGED[name]
    banner(f"sparse_mlp clamp / bad indices {name}")
    L = synth.make_layer(cfg, DEV, with_kv=False)
    y = synth.make_y(cfg, DEV)
    F = cfg.F
    S = np.array([3, 10, F // 2, F - 1])
    # the device count says 9 but the capacity is 4: only the 4 slots are read
    idx = i32(S)
    cnt = i32([9])
    out = torch.empty((cfg.batch, cfg.d), dtype=torch.float32, device=DEV)
    ws = dv.workspace(dv.OP_SPARSE_MLP, batch=cfg.batch, d=cfg.d, max_count_m=4)
    dv.sparse_mlp(y, L.W1t, L.W2t, idx, cnt, 4, out, 0, ws)
    ref = O.sparse_mlp(host(y), host(L.W1t), host(L.W2t), S)
    assert_close(out.cpu().numpy(), ref, TIGHT_MLP, "clamped count")
    # out-of-range entries contribute nothing
    idx = i32([3, -1, 10, F, F // 2, 1 << 30, F - 1])
    cnt = i32([7])
    ws = dv.workspace(dv.OP_SPARSE_MLP, batch=cfg.batch, d=cfg.d, max_count_m=7)
    dv.sparse_mlp(y, L.W1t, L.W2t, idx, cnt, 7, out, 0, ws)
    assert_close(out.cpu().numpy(), ref, TIGHT_MLP, "bad indices skipped")


# --------------------------------------------------------------------------- #
# A4 sparse MHA                                                               #
# --------------------------------------------------------------------------- #

def _mha_case(cfg, L, y, S, accumulate=False, cap=None, scale=None):
    B = y.shape[0]
    cap = len(S) if cap is None else cap
    scale = cfg.scale if scale is None else scale
    heads, cnt = put_set(S, cap)
    out = torch.full((B, cfg.d), 0.25 if accumulate else np.nan, dtype=torch.float32, device=DEV)
    ws = dv.workspace(dv.OP_SPARSE_MHA, batch=B, d=cfg.d, dh=cfg.dh, n_ctx=cfg.n_ctx,
                      max_count_a=cap)
    dv.sparse_mha(y, L.Wq, L.Wo, L.K, L.V, heads, cnt, cap, scale, out, accumulate, ws)
    ref = O.sparse_mha(host(y), host(L.Wq), host(L.Wo), host(L.K), host(L.V), S, scale)
    ref = ref + (0.25 if accumulate else 0.0)
    out2 = torch.full_like(out, 0.25 if accumulate else np.nan)
    dv.sparse_mha(y, L.Wq, L.Wo, L.K, L.V, heads, cnt, cap, scale, out2, accumulate, ws)
    assert torch.equal(out, out2), "sparse_mha not deterministic"
    return out.cpu().numpy(), ref


@pytest.mark.parametrize("name", SMALL + FULL)
def test_sparse_mha_parity(name):
    cfg = cfg_of(name)
    banner(f"sparse_mha {name}")
    L = synth.make_layer(cfg, DEV)
    y = synth.make_y(cfg, DEV)
    S = synth.random_index_set(cfg.h, cfg.k_a, seed=cfg.cfg_id + 1).numpy()
    got, ref = _mha_case(cfg, L, y, S)
    assert_close(got, ref, tol_of(cfg, TIGHT_ATTN), f"mha {name}")


@pytest.mark.parametrize("name", ["c1", "bf16-ragged", "f32-ragged", "long-ctx", "mixed-kv", "b17"])
def test_sparse_mha_edges(name):
    cfg = cfg_of(name)
    banner(f"sparse_mha edges {name}")
    L = synth.make_layer(cfg, DEV)
    y = synth.make_y(cfg, DEV)
    tol = tol_of(cfg, TIGHT_ATTN)
    got, _ = _mha_case(cfg, L, y, np.zeros(0, dtype=np.int64), cap=2)
    assert np.array_equal(got, np.zeros_like(got)), "no heads must give exact zero"
    got, ref = _mha_case(cfg, L, y, np.arange(cfg.h))
    assert_close(got, ref, tol, "mha all heads")
    got, ref = _mha_case(cfg, L, y, np.array([cfg.h - 1]), accumulate=True)
    assert_close(got, ref, tol, "mha last head accumulate")
    got, ref = _mha_case(cfg, L, y, np.array([0]), scale=1.0 / np.sqrt(cfg.dh))
    assert_close(got, ref, tol, "mha scaled")


# --------------------------------------------------------------------------- #
# A5 decode layer with the look-ahead predictor                               #
# --------------------------------------------------------------------------- #

def _layer_case(cfg, batch=None, with_next=True, seed_sets=None, act="relu", fp8=False):
    B = cfg.batch if batch is None else batch
    L = synth.make_layer(cfg, DEV, batch=B)
    row_scales = None
    if fp8:
        # weight-only fp8: W1t, W2t, W^Q, W^O as E4M3 codes with one scale per row
        q = {k: synth.quantize_rows_e4m3(getattr(L, k)) for k in ("W1t", "W2t", "Wq", "Wo")}
        for k, (codes, _) in q.items():
            setattr(L, k, codes)
        row_scales = tuple(q[k][1] for k in ("W1t", "W2t", "Wq", "Wo"))
    P1 = synth.make_predictor(cfg, DEV, layer=1)
    y = synth.make_y(cfg, DEV, batch=B)
    Lh = {k: host(v) for k, v in vars(L).items() if isinstance(v, torch.Tensor)}
    yh = host(y)
    # this layer's sets: the oracle's look-ahead sets from its own predictor on y
    S_M = O.predict_and_select(yh, Lh["A_M"], Lh["B_M"], cfg.k_m, True)
    S_A = O.predict_and_select(yh, Lh["A_A"], Lh["B_A"], cfg.k_a, True)
    cap_m, cap_a = min(cfg.F, B * cfg.k_m), min(cfg.h, B * cfg.k_a)
    idx_m, cnt_m = put_set(S_M, cap_m)
    idx_a, cnt_a = put_set(S_A, cap_a)
    layer = dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V, L.A_M, L.B_M, L.A_A, L.B_A,
                     k_m=cfg.k_m, k_a=cfg.k_a, scale=cfg.scale,
                     act=dv.DV_ACT_GELU if act == "gelu" else dv.DV_ACT_RELU,
                     row_scales=row_scales)
    nxt = dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V, P1["A_M"], P1["B_M"], P1["A_A"], P1["B_A"],
                   k_m=cfg.k_m, k_a=cfg.k_a, scale=cfg.scale) if with_next else None
    n_idx_m = torch.full((cap_m,), -9, dtype=torch.int32, device=DEV)
    n_idx_a = torch.full((cap_a,), -9, dtype=torch.int32, device=DEV)
    n_cnt_m = torch.full((1,), -9, dtype=torch.int32, device=DEV)
    n_cnt_a = torch.full((1,), -9, dtype=torch.int32, device=DEV)
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=cap_m, max_count_a=cap_a)
    y_out = torch.full_like(y, np.nan)
    dv.decode_layer(layer, nxt, y, y_out, idx_m, cnt_m, cap_m, idx_a, cnt_a, cap_a,
                    n_idx_m, n_cnt_m, n_idx_a, n_cnt_a, ws)
    torch.cuda.synchronize()
    layer_d = dict(W1t=Lh["W1t"], W2t=Lh["W2t"], Wq=Lh["Wq"], Wo=Lh["Wo"], K=Lh["K"], V=Lh["V"],
                   act=act)
    if fp8:
        for k, sc in zip(("W1t", "W2t", "Wq", "Wo"), row_scales):
            layer_d[k] = O.Fp8Rows(Lh[k], host(sc))
    y_ref, _ = O.decode_layer(yh, layer_d, S_M, S_A, None, cfg.scale)
    res = dict(y_out=y_out.cpu().numpy(), y_ref=y_ref, y=y, layer=layer, ws=ws)
    if with_next:
        P1h = {k: host(v) for k, v in P1.items()}
        res["sets"] = []
        for A, Bm, k, ni, nc in ((P1h["A_M"], P1h["B_M"], cfg.k_m, n_idx_m, n_cnt_m),
                                 (P1h["A_A"], P1h["B_A"], cfg.k_a, n_idx_a, n_cnt_a)):
            c = int(nc.cpu()[0])
            got = ni.cpu().numpy()[:c]
            ref_s = O.predict_scores(yh, A, Bm)
            res["sets"].append((got, ref_s, k, score_bound(yh, A, Bm)))
        # the same call again must give bit-identical results
        y2 = torch.full_like(y, np.nan)
        dv.decode_layer(layer, nxt, y, y2, idx_m, cnt_m, cap_m, idx_a, cnt_a, cap_a,
                        n_idx_m, n_cnt_m, n_idx_a, n_cnt_a, ws)
        assert torch.equal(y2, y_out), "decode_layer not deterministic"
    return res


@pytest.mark.parametrize("name", SMALL + FULL)
def test_decode_layer_parity(name):
    cfg = cfg_of(name)
    banner(f"decode_layer {name}")
    r = _layer_case(cfg)
    assert_close(r["y_out"], r["y_ref"], tol_of(cfg, TIGHT_ATTN), f"layer {name}")
    for got, ref_s, k, bound in r["sets"]:
        check_sets_certified(got, ref_s, k, True, bound, f"{name} next sets")


@pytest.mark.parametrize("name", ["bf16-ragged", "c4"])
def test_decode_layer_gelu(name):
    """A layer whose MLP uses GeLU: output and the next layer's sets (the predictor does
    not depend on the activation); c4 at batch 1 is the benchmarked shape."""
    cfg = cfg_of(name)
    banner(f"decode_layer gelu {name}")
    r = _layer_case(cfg, batch=1 if name == "c4" else None, act="gelu")
    assert_close(r["y_out"], r["y_ref"], tol_of(cfg, TIGHT_ATTN), f"gelu layer {name}")
    for got, ref_s, k, bound in r["sets"]:
        check_sets_certified(got, ref_s, k, True, bound, f"gelu {name} next sets")


FP8_CASES = {
    "c1": CONFIGS["c1"], "bf16-dh256": RAGGED["bf16-dh256"],
    "fp8-ragged": LayerConfig("fp8-ragged", 17, d=272, F=1000, h=6, dh=64, batch=3, n_ctx=37,
                              k_m=97, k_a=2, r=24, union=True),
    "c2": CONFIGS["c2"], "c3": CONFIGS["c3"],
}


@pytest.mark.parametrize("name", list(FP8_CASES) + ["c4"])
def test_decode_layer_fp8(name):
    """Weight-only fp8 layers (E4M3 rows, per-row scales): the oracle computes with the
    exactly dequantized weights; c4 at batch 1 is the benchmarked shape."""
    cfg = FP8_CASES.get(name, CONFIGS.get(name))
    banner(f"decode_layer fp8 {name}")
    r = _layer_case(cfg, batch=1 if name == "c4" else None, fp8=True)
    tol = BOUND_F32 * 10 if cfg.wdtype == "f32" else TIGHT_ATTN
    assert_close(r["y_out"], r["y_ref"], tol, f"fp8 layer {name}")
    for got, ref_s, k, bound in r["sets"]:
        check_sets_certified(got, ref_s, k, True, bound, f"fp8 {name} next sets")


@pytest.mark.parametrize("name", ["fp8-ragged", "c2", "c4"])
def test_decode_layer_fp8_last_layer(name):
    """fp8 layers without a next layer: at c4 batch 1 (the benchmarked sparse MLP + MHA)
    the attention and the waiting fp8 row sum share one launch."""
    cfg = FP8_CASES.get(name, CONFIGS.get(name))
    banner(f"decode_layer fp8 last layer {name}")
    r = _layer_case(cfg, batch=1 if name == "c4" else None, with_next=False, fp8=True)
    tol = BOUND_F32 * 10 if cfg.wdtype == "f32" else TIGHT_ATTN
    assert_close(r["y_out"], r["y_ref"], tol, f"fp8 last layer {name}")


def test_decode_layer_last_layer_and_alias():
    cfg = RAGGED["bf16-ragged"]
    banner("decode_layer last layer, y_out aliasing y_in")
    r = _layer_case(cfg, with_next=False)
    assert_close(r["y_out"], r["y_ref"], TIGHT_ATTN, "last layer")
    y = r["y"].clone()
    L = synth.make_layer(cfg, DEV)
    S_M = np.arange(0, cfg.F, 9)
    S_A = np.array([1, 4])
    idx_m, cnt_m = put_set(S_M, len(S_M))
    idx_a, cnt_a = put_set(S_A, 2)
    ref, _ = O.decode_layer(host(y), dict(W1t=host(L.W1t), W2t=host(L.W2t), Wq=host(L.Wq),
                                          Wo=host(L.Wo), K=host(L.K), V=host(L.V)),
                            S_M, S_A, None)
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=cfg.batch, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=len(S_M), max_count_a=2)
    layer = dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V)
    dv.decode_layer(layer, None, y, y, idx_m, cnt_m, len(S_M), idx_a, cnt_a, 2,
                    None, None, None, None, ws)
    assert_close(y.cpu().numpy(), ref, TIGHT_ATTN, "in place")


def test_decode_layer_lookahead_uses_input():
    """The next layer's sets come from y_in: with a predictor that sees y_in and
    y_out differently, the GPU sets must match the y_in ones."""
    cfg = RAGGED["c1"]
    banner("decode_layer look-ahead differential")
    r = _layer_case(cfg)
    y_in = host(r["y"])
    y_out = r["y_out"]
    for (got, ref_s, k, bound) in r["sets"]:
        check_sets_certified(got, ref_s, k, True, bound, "sets from y_in")
    # the sets that y_out would give differ, so the check above is not vacuous
    P1 = synth.make_predictor(cfg, "cpu", layer=1)
    s_in = O.predict_and_select(y_in, host(P1["A_M"]), host(P1["B_M"]), cfg.k_m, True)
    s_out = O.predict_and_select(y_out, host(P1["A_M"]), host(P1["B_M"]), cfg.k_m, True)
    assert not np.array_equal(s_in, s_out)


# Shapes that route the single attention + waiting row-sum launch (a layer without a
# next layer) through its per-slot path: with one 256-column slice, the W2 share of a
# chunk is more than one tile (12000 rows over 19 chunks), so the blocks take their
# W^O rows one head slot at a time, each slot waited for by one thread, and the key
# splits combine o themselves.
WAIT_SHAPES = {
    "slot-path": LayerConfig("slot-path", 31, d=256, F=32768, h=4, dh=64, batch=1, n_ctx=300,
                             k_m=12000, k_a=3, r=16),
    "slot-path-b2": LayerConfig("slot-path-b2", 32, d=256, F=32768, h=4, dh=64, batch=2,
                                n_ctx=300, k_m=12000, k_a=3, r=16, union=True),
}


@pytest.mark.parametrize("name", list(WAIT_SHAPES))
def test_decode_layer_waiting_slot_path(name):
    cfg = WAIT_SHAPES[name]
    banner(f"decode_layer waiting launch, per-slot path {name}")
    dv.timing_read(16)
    dv.timing_enable(True)
    try:
        r = _layer_case(cfg, with_next=False)
    finally:
        dv.timing_enable(False)
    _, launches = dv.timing_read(16)
    # the plan under test: the row dots, then the single waiting launch
    assert len(launches) == 2, f"{name}: {len(launches)} launches, expected the two-launch plan"
    assert_close(r["y_out"], r["y_ref"], TIGHT_ATTN, f"per-slot path {name}")


@pytest.mark.parametrize("B,fp8,expected", [(1, False, 2), (2, False, 3), (1, True, 2)])
def test_sparse_step_launch_plan(B, fp8, expected):
    """The OPT-175B-shaped sparse step (no next layer) takes the row dots plus the single
    waiting launch at one token (bf16 or fp8 rows), and three launches (row dots,
    attention, row sum) at two tokens, where fewer than two row-sum blocks per CU would
    fit beside the attention."""
    cfg = CONFIGS["c4"]
    banner(f"sparse step launch plan c4 batch {B} fp8={fp8}")
    L = synth.make_layer(cfg, DEV, batch=B)
    y = synth.make_y(cfg, DEV, batch=B)
    cap_m, cap_a = min(cfg.F, B * cfg.k_m), min(cfg.h, B * cfg.k_a)
    idx_m, cnt_m = put_set(synth.random_index_set(cfg.F, cap_m, seed=81 + B).numpy(), cap_m)
    idx_a, cnt_a = put_set(synth.random_index_set(cfg.h, cap_a, seed=91 + B).numpy(), cap_a)
    row_scales = None
    if fp8:
        q = {k: synth.quantize_rows_e4m3(getattr(L, k)) for k in ("W1t", "W2t", "Wq", "Wo")}
        for k, (codes, _) in q.items():
            setattr(L, k, codes)
        row_scales = tuple(q[k][1] for k in ("W1t", "W2t", "Wq", "Wo"))
    layer = dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V, k_m=cfg.k_m, k_a=cfg.k_a, scale=cfg.scale,
                     row_scales=row_scales)
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=cap_m, max_count_a=cap_a)
    y_out = torch.full_like(y, np.nan)
    dv.timing_read(16)
    dv.timing_enable(True)
    try:
        dv.decode_layer(layer, None, y, y_out, idx_m, cnt_m, cap_m, idx_a, cnt_a, cap_a,
                        None, None, None, None, ws)
        torch.cuda.synchronize()
    finally:
        dv.timing_enable(False)
    _, launches = dv.timing_read(16)
    assert len(launches) == expected, f"batch {B}: {len(launches)} launches, expected {expected}"
    assert torch.isfinite(y_out).all(), f"batch {B}: non-finite output"


@pytest.mark.parametrize("name", ["bf16-ragged", "c4"])
def test_decode_layer_waiting_bad_heads(name):
    """The single waiting launch with a head list holding an index outside [0, h) and a
    count below capacity: the bad head contributes nothing (its W^O rows are skipped,
    its slot still reported complete, so no wait gives up), slots past the count are
    never waited for, and the output equals the oracle's over the valid heads."""
    cfg = cfg_of(name)
    B = 1
    banner(f"decode_layer waiting launch, bad head index {name}")
    L = synth.make_layer(cfg, DEV, batch=B)
    y = synth.make_y(cfg, DEV, batch=B)
    S_M = synth.random_index_set(cfg.F, cfg.k_m, seed=cfg.cfg_id + 71).numpy()
    S_A = synth.random_index_set(cfg.h, min(cfg.k_a, cfg.h - 1), seed=cfg.cfg_id + 72).numpy()
    listed = np.concatenate([S_A[:1], [cfg.h + 3], S_A[1:]]).astype(np.int32)
    cap_a = len(listed) + 2                                  # count below capacity
    idx_m, cnt_m = put_set(S_M, len(S_M))
    idx_a = torch.full((cap_a,), 7, dtype=torch.int32, device=DEV)
    idx_a[:len(listed)] = torch.as_tensor(listed, device=DEV)
    cnt_a = torch.tensor([len(listed)], dtype=torch.int32, device=DEV)
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=len(S_M), max_count_a=cap_a)
    layer = dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V, scale=cfg.scale)
    y_out = torch.full_like(y, np.nan)
    dv.decode_layer(layer, None, y, y_out, idx_m, cnt_m, len(S_M), idx_a, cnt_a, cap_a,
                    None, None, None, None, ws)
    dv.check()
    ref, _ = O.decode_layer(host(y), dict(W1t=host(L.W1t), W2t=host(L.W2t), Wq=host(L.Wq),
                                          Wo=host(L.Wo), K=host(L.K), V=host(L.V)),
                            S_M, np.sort(S_A), None, cfg.scale)
    assert_close(y_out.cpu().numpy(), ref, TIGHT_ATTN, f"bad head {name}")


@pytest.mark.parametrize("batch", [1, 2, 4, 8, 16])
def test_decode_layer_c4(batch):
    """The OPT-175B-shaped layer at full size, at every batch of the workload (batch 1
    is the benchmarked launch; 4 and 8 take the five-launch look-ahead step, the row
    dots with the row length split into parts and a partly filled 16-token tile)."""
    cfg = CONFIGS["c4"]
    banner(f"decode_layer c4 batch={batch}")
    r = _layer_case(cfg, batch=batch)
    assert_close(r["y_out"], r["y_ref"], TIGHT_ATTN, f"c4 B={batch}")
    swaps = 0
    for got, ref_s, k, bound in r["sets"]:
        swaps += check_sets_certified(got, ref_s, k, True, bound, f"c4 B={batch} next sets")
    print(f"c4 B={batch}: certified boundary swaps {swaps}")


def test_workspace_shared_across_calls():
    """One workspace serves different entry points in turn (its contents left by one
    call are never read by the next): results equal those of fresh workspaces."""
    cfg = cfg_of("c2")
    banner("shared workspace c2")
    L = synth.make_layer(cfg, DEV)
    y = synth.make_y(cfg, DEV)
    S_M = synth.random_index_set(cfg.F, cfg.k_m, seed=5).numpy()
    S_A = synth.random_index_set(cfg.h, cfg.k_a, seed=6).numpy()
    idx_m, cnt_m = put_set(S_M, len(S_M))
    idx_a, cnt_a = put_set(S_A, len(S_A))
    shared = torch.full((max(
        dv.workspace_bytes(dv.OP_SPARSE_MLP, batch=1, d=cfg.d, max_count_m=len(S_M)),
        dv.workspace_bytes(dv.OP_SPARSE_MHA, batch=1, d=cfg.d, dh=cfg.dh, n_ctx=cfg.n_ctx,
                           max_count_a=len(S_A)),
        dv.workspace_bytes(dv.OP_PREDICT, batch=1, d=cfg.d, r=cfg.r, N=cfg.F)),), 0xA5,
        dtype=torch.uint8, device=DEV)
    outs = {}
    for tag, ws_of in (("fresh", None), ("shared", shared)):
        for rep in range(2):
            o_m = torch.empty((1, cfg.d), dtype=torch.float32, device=DEV)
            ws = ws_of if ws_of is not None else dv.workspace(dv.OP_SPARSE_MLP, batch=1, d=cfg.d,
                                                              max_count_m=len(S_M))
            dv.sparse_mlp(y, L.W1t, L.W2t, idx_m, cnt_m, len(S_M), o_m, 0, ws)
            o_a = torch.empty((1, cfg.d), dtype=torch.float32, device=DEV)
            ws = ws_of if ws_of is not None else dv.workspace(
                dv.OP_SPARSE_MHA, batch=1, d=cfg.d, dh=cfg.dh, n_ctx=cfg.n_ctx,
                max_count_a=len(S_A))
            dv.sparse_mha(y, L.Wq, L.Wo, L.K, L.V, idx_a, cnt_a, len(S_A), cfg.scale, o_a, 0, ws,
                          h=cfg.h, dh=cfg.dh)
            sc = torch.empty((1, cfg.F), dtype=torch.float32, device=DEV)
            ws = ws_of if ws_of is not None else dv.workspace(dv.OP_PREDICT, batch=1, d=cfg.d,
                                                              r=cfg.r, N=cfg.F)
            dv.predict(y, L.A_M, L.B_M, sc, ws)
            outs[(tag, rep)] = (o_m, o_a, sc)
    for a, b in zip(outs[("fresh", 0)], outs[("shared", 1)]):
        assert torch.equal(a, b)
