"""The 24-layer OPT-175B-shaped stack at batch 32 (the largest configuration), end to
end on the GPU through dv_decode_layer with the look-ahead predictor, checked against
the oracle layer by layer (teacher forcing: the oracle starts each checked layer from
the GPU's own input and index sets).

What one GPU holds: 24 layers of bf16 weights (W1t, W2t, W^Q, W^O, the predictor) plus
each layer's bf16 KV cache for 32 sequences of 2048 tokens, about 155 GB of HBM.

Checks at layers 0, 12 and 23:
  - the layer output of all 32 tokens (both 16-token groups of the matrix-core tiles);
  - the union sets the layer predicted for the next layer, against the oracle's
    scores for all 32 tokens (certified boundary swaps only).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from contextual_sparsity_mlp_amd import dv, synth
from contextual_sparsity_mlp_amd.synth import CONFIGS
from gpu_helpers import TIGHT_ATTN, assert_close, banner, check_sets_certified, host, score_bound
from oracle import dv_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"
CHECK_LAYERS = (0, 12, 23)


@pytest.mark.timeout(900)
def test_decode_stack_c5_teacher_forced():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cfg = CONFIGS["c5"]
    B, nl = cfg.batch, cfg.layers
    banner(f"decode stack c5: generating {nl} layers, batch {B}")
    layers = [synth.make_layer(cfg, DEV, layer=l, batch=B) for l in range(nl)]
    dvl = [dv.Layer(L.W1t, L.W2t, L.Wq, L.Wo, L.K, L.V, L.A_M, L.B_M, L.A_A, L.B_A,
                    k_m=cfg.k_m, k_a=cfg.k_a, scale=cfg.scale) for L in layers]
    y = synth.make_y(cfg, DEV, batch=B)
    cap_m, cap_a = min(cfg.F, B * cfg.k_m), min(cfg.h, B * cfg.k_a)
    i32 = lambda n: torch.full((n,), -9, dtype=torch.int32, device=DEV)  # noqa: E731
    sets = [dict(m=i32(cap_m), cm=i32(1), a=i32(cap_a), ca=i32(1)) for _ in range(2)]
    ws = dv.workspace(dv.OP_DECODE_LAYER, batch=B, d=cfg.d, F=cfg.F, h=cfg.h, dh=cfg.dh,
                      n_ctx=cfg.n_ctx, r=cfg.r, max_count_m=cap_m, max_count_a=cap_a)

    # layer 0's sets from its own predictor (nothing runs ahead of it)
    s_m = torch.empty((B, cfg.F), dtype=torch.float32, device=DEV)
    s_a = torch.empty((B, cfg.h), dtype=torch.float32, device=DEV)
    wsp = dv.workspace(dv.OP_PREDICT, batch=B, d=cfg.d, r=cfg.r, N=cfg.F)
    wst = dv.workspace(dv.OP_SELECT_TOPK, batch=B, N=cfg.F)
    dv.predict(y, layers[0].A_M, layers[0].B_M, s_m, wsp)
    dv.select_topk(s_m, cfg.k_m, 1, sets[0]["m"], sets[0]["cm"], wst)
    dv.predict(y, layers[0].A_A, layers[0].B_A, s_a, wsp)
    dv.select_topk(s_a, cfg.k_a, 1, sets[0]["a"], sets[0]["ca"], wst)

    saved = {}
    y_cur = y.clone()
    y_nxt = torch.empty_like(y)
    for l in range(nl):
        si, so = sets[l % 2], sets[(l + 1) % 2]
        if l in CHECK_LAYERS:
            torch.cuda.synchronize()
            c_m, c_a = int(si["cm"].cpu()[0]), int(si["ca"].cpu()[0])
            saved[l] = dict(y=host(y_cur), S_M=si["m"].cpu().numpy()[:c_m].copy(),
                            S_A=si["a"].cpu().numpy()[:c_a].copy())
        nx = dvl[l + 1] if l + 1 < nl else None
        dv.decode_layer(dvl[l], nx, y_cur, y_nxt, si["m"], si["cm"], cap_m, si["a"], si["ca"],
                        cap_a, so["m"] if nx else None, so["cm"] if nx else None,
                        so["a"] if nx else None, so["ca"] if nx else None, ws)
        if l in CHECK_LAYERS:
            torch.cuda.synchronize()
            saved[l]["y_out"] = y_nxt.cpu().numpy().copy()
            if nx is not None:
                c_m, c_a = int(so["cm"].cpu()[0]), int(so["ca"].cpu()[0])
                saved[l]["next"] = (so["m"].cpu().numpy()[:c_m].copy(),
                                    so["a"].cpu().numpy()[:c_a].copy())
        y_cur, y_nxt = y_nxt, y_cur
    torch.cuda.synchronize()
    assert np.all(np.isfinite(y_cur.cpu().numpy())), "stack output not finite"

    for l in CHECK_LAYERS:
        banner(f"decode stack c5: oracle check of layer {l}")
        sv = saved[l]
        L = layers[l]
        # every layer's sets are unions of per-token top-k: sizes within [k, B k]
        assert cfg.k_m <= len(sv["S_M"]) <= cap_m and cfg.k_a <= len(sv["S_A"]) <= cap_a
        ld = dict(W1t=host(L.W1t), W2t=host(L.W2t), Wq=host(L.Wq), Wo=host(L.Wo),
                  K=host(L.K), V=host(L.V))
        y_ref, _ = O.decode_layer(sv["y"], ld, sv["S_M"], sv["S_A"], None, cfg.scale)
        e = assert_close(sv["y_out"], y_ref, TIGHT_ATTN, f"c5 layer {l}")
        print(f"c5 layer {l}: |S_M|={len(sv['S_M'])} |S_A|={len(sv['S_A'])} rel err {e:.2e}")
        del ld
        if "next" in sv:
            P = layers[l + 1]
            for (A, Bm, k, got) in ((P.A_M, P.B_M, cfg.k_m, sv["next"][0]),
                                    (P.A_A, P.B_A, cfg.k_a, sv["next"][1])):
                Ah, Bh = host(A), host(Bm)
                ref_s = O.predict_scores(sv["y"], Ah, Bh)
                swaps = check_sets_certified(got, ref_s, k, True, score_bound(sv["y"], Ah, Bh),
                                             f"c5 layer {l} next sets")
                print(f"c5 layer {l}: next set size {len(got)}, certified swaps {swaps}")
