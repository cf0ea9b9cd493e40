"""Byte accounting used by the benchmark, pinned to the survey-notes page's KV-cache
sizing example and to the sizes the configs imply."""
from conftest import load_golden

from contextual_sparsity_mlp_amd import accounting as A
from contextual_sparsity_mlp_amd.synth import CONFIGS


def test_kv_bytes_example():
    g = load_golden("kv_bytes.json")
    per = A.kv_bytes_per_token(g["hidden"], g["layers"], g["bytes_per_elem"])
    assert per == g["per_token_bytes"]
    assert per * g["tokens"] == g["total_bytes"]


def test_c4_batch1_bytes():
    c = CONFIGS["c4"]
    b = A.step_bytes(batch=1, d=c.d, F=c.F, h=c.h, dh=c.dh, n_ctx=c.n_ctx, r=c.r, u_m=c.k_m,
                     u_a=c.k_a)
    # 4915 neurons x 2 rows x 12288 x 2 B; 19 heads x 2 x 128 rows x 12288 x 2 B;
    # 19 heads x 2 x 2048 tokens x 128 x 2 B
    assert b.mlp == 4915 * 2 * 12288 * 2 == 241_582_080
    assert b.attn_weights == 19 * 2 * 128 * 12288 * 2
    assert b.kv == 19 * 2 * 2048 * 128 * 2
    assert b.predictor == (2 * 12288 * 1000 + 1000 * 49152 + 1000 * 96) * 2
    # the KV of one selected head and token matches the per-token formula for one layer
    assert b.kv == A.kv_bytes_per_token(c.dh, 1) * c.n_ctx * c.k_a
    ph = A.phase_bytes(batch=1, d=c.d, F=c.F, h=c.h, dh=c.dh, n_ctx=c.n_ctx, r=c.r, u_m=c.k_m,
                       u_a=c.k_a)
    # the three launches together move every algorithmic byte of the step once, plus
    # y read a second time and the scores read by the top-k
    assert sum(ph) == b.total + 1 * c.d * 4 + (c.F + c.h) * 4
    sp = A.phase_bytes(batch=1, d=c.d, F=c.F, h=c.h, dh=c.dh, n_ctx=c.n_ctx, r=c.r, u_m=c.k_m,
                       u_a=c.k_a, with_predictor=False)
    # the sparse layer alone: two launches, y read twice
    assert len(sp) == 2 and sum(sp) == b.selected + 1 * c.d * 4
    sp3 = A.phase_bytes(batch=1, d=c.d, F=c.F, h=c.h, dh=c.dh, n_ctx=c.n_ctx, r=c.r, u_m=c.k_m,
                        u_a=c.k_a, with_predictor=False, sparse_launches=3)
    # attention in a launch of its own: the same bytes, split three ways
    assert len(sp3) == 3 and sum(sp3) == sum(sp) and sp3[0] == sp[0]
    sp1 = A.phase_bytes(batch=1, d=c.d, F=c.F, h=c.h, dh=c.dh, n_ctx=c.n_ctx, r=c.r, u_m=c.k_m,
                        u_a=c.k_a, with_predictor=False, sparse_launches=1)
    # everything in one launch: exactly the step's bytes, y read once
    assert sp1 == [b.selected]
    # the KV append: W^K, W^V in full plus the written rows, one more cached row attended
    kw = dict(batch=2, d=c.d, F=c.F, h=c.h, dh=c.dh, n_ctx=c.n_ctx, r=c.r, u_m=c.k_m, u_a=c.k_a)
    ba, b0 = A.step_bytes(**kw, kv_append=True), A.step_bytes(**kw)
    assert ba.total - b0.total == 2 * c.d * c.d * 2 + 2 * 2 * c.d * 2 + 2 * c.k_a * 2 * c.dh * 2
    pa = A.phase_bytes(**kw, kv_append=True)
    assert sum(pa) - sum(A.phase_bytes(**kw)) == ba.total - b0.total
    # five look-ahead launches (a batch on the matrix cores): the attention and the
    # predictor B factors apart, and the score histograms reading the scores once more
    kw16 = dict(kw, batch=16)
    p3, p5 = A.phase_bytes(**kw16), A.phase_bytes(**kw16, lookahead_launches=5)
    assert len(p5) == 5 and p5[0] == p3[0] and p5[4] == p3[2]
    assert p5[1] + p5[2] == p3[1]
    assert sum(p5) == sum(p3) + 16 * (c.F + c.h) * 4


def test_flops_intensity_batch1():
    c = CONFIGS["c4"]
    kw = dict(d=c.d, F=c.F, h=c.h, dh=c.dh, n_ctx=c.n_ctx, r=c.r, u_m=c.k_m, u_a=c.k_a)
    f = A.step_flops(batch=1, **kw)
    b = A.step_bytes(batch=1, **kw).total
    assert 0.9 < f / b < 1.1      # about one flop per byte at batch 1: bound by HBM
