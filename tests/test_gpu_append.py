"""The full decode step with the KV append, through dv_decode_layer, against the oracle
(KV-cache blog page, figure (b): the current token's key and value join the cache
and are attended with it; every head's row is stored).

Checked on each case:
  * the layer output against the oracle's step over the n + 1 rows;
  * the stored row n of every (token, head) against the exact y W^K, y W^V: within
    one rounding to the cache's type of the fp32 dot product, and (bf16 caches) equal
    to the oracle's rounded row in all but boundary cases;
  * every other cache row bit-identical to what it held before;
  * the next layer's sets (look-ahead), and a repeated call bit-identical.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from contextual_sparsity_mlp_amd import dv, synth
from contextual_sparsity_mlp_amd.synth import CONFIGS, LayerConfig
from gpu_helpers import (BOUND_F32, TIGHT_ATTN, assert_close, banner, check_sets_certified, host,
                         score_bound)
from oracle import dv_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"
FILL = 1.0e4          # spare cache rows hold this; no computed row takes it

CASES = {
    "c1": CONFIGS["c1"],
    "bf16-ragged": LayerConfig("bf16-ragged", 11, d=264, F=1000, h=6, dh=64, batch=3, n_ctx=37,
                               k_m=97, k_a=2, r=24, union=True),
    "f32-ragged": LayerConfig("f32-ragged", 12, d=72, F=300, h=5, dh=32, batch=2, n_ctx=5,
                              k_m=31, k_a=3, r=7, wdtype="f32", kvdtype="f32", union=True),
    "mixed-kv": LayerConfig("mixed-kv", 15, d=256, F=1024, h=4, dh=64, batch=5, n_ctx=130,
                            k_m=100, k_a=2, r=32, kvdtype="f32", union=True),
    "c2": CONFIGS["c2"], "c3": CONFIGS["c3"], "c4": CONFIGS["c4"],
}


def _set(S, cap):
    buf = torch.full((max(cap, 1),), -1, dtype=torch.int32, device=DEV)
    if len(S):
        buf[: len(S)] = torch.as_tensor(np.asarray(S, dtype=np.int32), device=DEV)
    return buf, torch.as_tensor(np.array([len(S)], dtype=np.int32), device=DEV)


def _widen(a):
    return O.widen(a)


def _append_case(cfg, batch=None, n=None, with_next=False, fp8=False, spare=3):
    """One decode step with the append at row n (default: the config's cache length)."""
    B = cfg.batch if batch is None else batch
    n = cfg.n_ctx if n is None else n
    L = synth.make_layer(cfg, DEV, batch=B, with_kv=False)
    Wk, Wv = synth.make_kv_weights(cfg, DEV)
    # a cache of n seeded rows and `spare` rows of FILL
    K, V = synth.make_kv_cache(dataclasses.replace(cfg, n_ctx=n), n + spare, DEV, batch=B,
                               fill=FILL)
    row_scales = kv_scales = None
    W = dict(W1t=L.W1t, W2t=L.W2t, Wq=L.Wq, Wo=L.Wo, Wk=Wk, Wv=Wv)
    scales = {}
    if fp8:
        for k in W:
            W[k], scales[k] = synth.quantize_rows_e4m3(W[k])
        row_scales = tuple(scales[k] for k in ("W1t", "W2t", "Wq", "Wo"))
        kv_scales = (scales["Wk"], scales["Wv"])
    y = synth.make_y(cfg, DEV, batch=B)
    yh = host(y)
    Ah = {k: host(getattr(L, k)) for k in ("A_M", "B_M", "A_A", "B_A")}
    S_M = O.predict_and_select(yh, Ah["A_M"], Ah["B_M"], cfg.k_m, True)
    S_A = O.predict_and_select(yh, Ah["A_A"], Ah["B_A"], cfg.k_a, True)
    cap_m, cap_a = min(cfg.F, B * cfg.k_m), min(cfg.h, B * cfg.k_a)
    idx_m, cnt_m = _set(S_M, cap_m)
    idx_a, cnt_a = _set(S_A, cap_a)
    layer = dv.Layer(W["W1t"], W["W2t"], W["Wq"], W["Wo"], K, V, L.A_M, L.B_M, L.A_A, L.B_A,
                     k_m=cfg.k_m, k_a=cfg.k_a, scale=cfg.scale, row_scales=row_scales,
                     Wk=W["Wk"], Wv=W["Wv"], kv_scales=kv_scales, n_ctx=n)
    P1 = synth.make_predictor(cfg, DEV, layer=1) if with_next else None
    nxt = dv.Layer(W["W1t"], W["W2t"], W["Wq"], W["Wo"], K, V, P1["A_M"], P1["B_M"], P1["A_A"],
                   P1["B_A"], k_m=cfg.k_m, k_a=cfg.k_a, scale=cfg.scale) if with_next else None
    n_idx_m = torch.full((cap_m,), -9, dtype=torch.int32, device=DEV)
    n_idx_a = torch.full((cap_a,), -9, dtype=torch.int32, device=DEV)
    n_cnt_m = torch.full((1,), -9, dtype=torch.int32, device=DEV)
    n_cnt_a = torch.full((1,), -9, dtype=torch.int32, device=DEV)
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=n, r=cfg.r, max_count_m=cap_m, max_count_a=cap_a)
    K0, V0 = host(K), host(V)
    y_out = torch.full_like(y, np.nan)
    dv.decode_layer(layer, nxt, y, y_out, idx_m, cnt_m, cap_m, idx_a, cnt_a, cap_a,
                    n_idx_m, n_cnt_m, n_idx_a, n_cnt_a, ws)
    torch.cuda.synchronize()
    K1, V1 = host(K), host(V)

    def stored(name):
        return O.Fp8Rows(host(W[name]), host(scales[name])) if fp8 else host(W[name])

    layer_d = {k: stored(k) for k in W}
    layer_d.update(K=K0, V=V0)
    y_ref, _, (k_row, v_row) = O.decode_layer_append(yh, layer_d, S_M, S_A, None, n, cfg.scale)
    res = dict(y_out=y_out.cpu().numpy(), y_ref=y_ref, n=n)

    # the stored rows: within one rounding of the fp32 dot product
    k_ex, v_ex = O.kv_for_token(yh, layer_d["Wk"], layer_d["Wv"])
    u_store = 2.0 ** -8 if K0.dtype == np.uint16 else 2.0 ** -24
    for nm, ex, got_all, ref_row in (("k", k_ex, K1, k_row), ("v", v_ex, V1, v_row)):
        Wabs = np.abs(_widen(layer_d["Wk" if nm == "k" else "Wv"]))
        mag = np.einsum("bd,icd->bic", np.abs(_widen(yh)), Wabs)          # sum_j |y_j||W_j|
        dot_err = 2.0 * cfg.d * 2.0 ** -24 * mag
        got = _widen(got_all[:, :, n])
        err = np.abs(got - ex)
        lim = u_store * np.abs(ex) + (1 + u_store) * dot_err
        assert np.all(err <= lim), \
            f"stored {nm} row: max excess {float(np.max(err - lim)):g} (row {n})"
        if K0.dtype == np.uint16:
            # bf16 spacing dwarfs the fp32 dot's error: both sides round to the same
            # bf16 value except next to a rounding boundary
            same = np.mean(got_all[:, :, n] == ref_row)
            assert same >= 0.98, f"stored {nm} row equals the oracle's rounding in only {same:.3%}"
            res[f"{nm}_same"] = same
    # every other row is untouched
    for nm, before, after in (("K", K0, K1), ("V", V0, V1)):
        assert np.array_equal(np.delete(after, n, axis=2), np.delete(before, n, axis=2)), \
            f"{nm}: rows other than {n} changed"

    if with_next:
        P1h = {k: host(v) for k, v in P1.items()}
        res["sets"] = []
        for A, Bm, k, ni, nc in ((P1h["A_M"], P1h["B_M"], cfg.k_m, n_idx_m, n_cnt_m),
                                 (P1h["A_A"], P1h["B_A"], cfg.k_a, n_idx_a, n_cnt_a)):
            c = int(nc.cpu()[0])
            res["sets"].append((ni.cpu().numpy()[:c], O.predict_scores(yh, A, Bm), k,
                                score_bound(yh, A, Bm)))
    # a repeated call rewrites the same row and gives the same output, bit for bit
    y2 = torch.full_like(y, np.nan)
    dv.decode_layer(layer, nxt, y, y2, idx_m, cnt_m, cap_m, idx_a, cnt_a, cap_a,
                    n_idx_m, n_cnt_m, n_idx_a, n_cnt_a, ws)
    torch.cuda.synchronize()
    assert torch.equal(y2, y_out), "decode step with the append not deterministic"
    assert np.array_equal(host(K), K1) and np.array_equal(host(V), V1), "append not deterministic"
    return res


def _tol(cfg):
    return BOUND_F32 * 10 if cfg.wdtype == "f32" else TIGHT_ATTN


@pytest.mark.parametrize("name,with_next", [
    ("c1", True), ("bf16-ragged", False), ("bf16-ragged", True), ("f32-ragged", True),
    ("mixed-kv", False), ("c2", True), ("c3", True)])
def test_append_parity(name, with_next):
    cfg = CASES[name]
    banner(f"decode_layer with KV append {name} next={with_next}")
    r = _append_case(cfg, with_next=with_next)
    assert_close(r["y_out"], r["y_ref"], _tol(cfg), f"append {name}")
    for got, ref_s, k, bound in r.get("sets", []):
        check_sets_certified(got, ref_s, k, True, bound, f"append {name} next sets")


@pytest.mark.parametrize("n", [0, 1, 63, 64, 127, 128, 129, 255])
def test_append_row_positions(n):
    """Empty cache (the current token alone), and rows around the key splits."""
    cfg = CASES["bf16-ragged"]
    banner(f"decode_layer with KV append at row {n}")
    r = _append_case(cfg, n=n, with_next=(n % 2 == 1))
    assert_close(r["y_out"], r["y_ref"], _tol(cfg), f"append at row {n}")


@pytest.mark.parametrize("with_next,fp8", [(False, False), (True, False), (True, True),
                                           (False, True)])
def test_append_opt175b_batch1(with_next, fp8):
    """The OPT-175B shape at batch 1: the appended rows of all 96 heads."""
    cfg = CASES["c4"]
    banner(f"decode_layer with KV append c4 batch 1 next={with_next} fp8={fp8}")
    r = _append_case(cfg, batch=1, with_next=with_next, fp8=fp8)
    assert_close(r["y_out"], r["y_ref"], TIGHT_ATTN, "append c4")
    for got, ref_s, k, bound in r.get("sets", []):
        check_sets_certified(got, ref_s, k, True, bound, "append c4 next sets")


def test_append_fp8_ragged():
    cfg = LayerConfig("fp8-ragged", 17, d=272, F=1000, h=6, dh=64, batch=3, n_ctx=37,
                      k_m=97, k_a=2, r=24, union=True)
    banner("decode_layer with KV append, fp8 ragged")
    r = _append_case(cfg, with_next=True, fp8=True)
    assert_close(r["y_out"], r["y_ref"], TIGHT_ATTN, "append fp8 ragged")


def test_append_steps_advance():
    """Three steps in a row: each appends at the next row and attends to the rows the
    earlier steps stored (the caller advances n_ctx)."""
    cfg = CASES["bf16-ragged"]
    B, n0 = cfg.batch, cfg.n_ctx
    banner("decode_layer with KV append, three steps")
    L = synth.make_layer(cfg, DEV, batch=B, with_kv=False)
    Wk, Wv = synth.make_kv_weights(cfg, DEV)
    K, V = synth.make_kv_cache(cfg, n0 + 4, DEV, batch=B, fill=FILL)
    S_M = np.arange(0, cfg.F, 7)
    S_A = np.array([1, 4])
    idx_m, cnt_m = _set(S_M, len(S_M))
    idx_a, cnt_a = _set(S_A, len(S_A))
    layer = dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, K, V, k_m=cfg.k_m, k_a=cfg.k_a, scale=cfg.scale,
                     Wk=Wk, Wv=Wv, n_ctx=n0)
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=n0 + 3, r=1, max_count_m=len(S_M), max_count_a=len(S_A))
    Wh = dict(W1t=host(L.W1t), W2t=host(L.W2t), Wq=host(L.Wq), Wo=host(L.Wo), Wk=host(Wk),
              Wv=host(Wv))
    Kh, Vh = host(K), host(V)
    y = synth.make_y(cfg, DEV, batch=B)
    for step in range(3):
        n = n0 + step
        layer.set_n_ctx(n)
        y_out = torch.empty_like(y)
        dv.decode_layer(layer, None, y, y_out, idx_m, cnt_m, len(S_M), idx_a, cnt_a, len(S_A),
                        None, None, None, None, ws)
        torch.cuda.synchronize()
        y_ref, _, (k_row, v_row) = O.decode_layer_append(host(y), dict(Wh, K=Kh, V=Vh), S_M, S_A,
                                                         None, n, cfg.scale)
        assert_close(y_out.cpu().numpy(), y_ref, TIGHT_ATTN, f"step {step}")
        # the oracle carries the GPU's stored rows forward (teacher forcing)
        Kh, Vh = host(K), host(V)
        y = y_out * 0.5
