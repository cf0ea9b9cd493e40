"""Checks that pin the CPU oracle to facts outside itself.

Each ``check_*`` takes the oracle module (or a patched copy of it) and raises
AssertionError on a mismatch.  ``test_oracle_pins.py`` runs them against the real
oracle; ``test_oracle_mutations.py`` runs them against oracles with a planted
mistake and requires that some check fails.

What pins what:
  * hand-worked examples in tests/golden (Deja Vu page, section 2.3, Eq. (1)
    and Eq. (2); predictor and look-ahead readings);
  * library routines for the dense special cases: torch.nn Linear-ReLU-Linear
    (the survey-notes page's FFN listing, bias zero) for S = all neurons, and
    torch scaled_dot_product_attention with concatenation and one output
    projection (the survey-notes page's projection listing) for S = all heads;
  * invariants: empty set gives 0, additivity over disjoint sets, the ReLU
    support reproduces the dense MLP, closed forms of softmax attention
    (n = 1, equal keys, one dominant logit);
  * the mean-shift restatement of a head on the Deja Vu page, section 3.2:
    H_i(y) = m_i(y) W_i^V with m_i a similarity-weighted mean of the x_j;
  * brute force: all k-subsets for top-k on tiny N, scalar loops for the
    products, np.lexsort for the ordering rule;
  * the KV-cache blog page, figure (b): a decode step over the cache plus the
    appended current token equals causal attention over the whole sequence.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch

from conftest import load_golden

RNG_SEED = 12345


def _rng(seed=RNG_SEED):
    return np.random.default_rng(seed)


def assert_close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"{what}: max err {err:g} > {tol:g} * {scale:g}"


# --------------------------------------------------------------------------- #
# golden, worked by hand                                                      #
# --------------------------------------------------------------------------- #

def check_golden_mlp(O):
    g = load_golden("mlp_tiny.json")
    for c in g["cases"]:
        out = O.sparse_mlp(np.array(g["y"]), np.array(g["W1t"]), np.array(g["W2t"]), c["S"])
        assert_close(out, c["out"], 1e-15, f"mlp S={c['S']}")


def check_golden_mha(O):
    g = load_golden("mha_tiny.json")
    for c in g["cases"]:
        out = O.sparse_mha(np.array(g["y"]), np.array(g["Wq"]), np.array(g["Wo"]),
                           np.array(g["K"]), np.array(g["V"]), c["S"], c["scale"])
        assert_close(out, c["out"], g["tol"], f"mha S={c['S']} scale={c['scale']}")


def check_golden_predictor(O):
    g = load_golden("predictor_tiny.json")
    s = O.predict_scores(np.array(g["y"]), np.array(g["A"]), np.array(g["Bm"]))
    assert_close(s, g["scores"], 1e-15, "scores")
    for c in g["topk"]:
        got = O.topk_row(np.array(g["scores"][0]), c["k"])
        assert list(got) == c["set"], f"topk k={c['k']}: {list(got)} != {c['set']}"
    for c in g["tie_cases"]:
        got = O.topk_row(np.array(c["scores"]), c["k"])
        assert list(got) == c["set"], f"ties {c['scores']} k={c['k']}: {list(got)}"
    for c in g["union_cases"]:
        got = O.select_sets(np.array(c["scores"]), c["k"], True)
        assert list(got) == c["set"], f"union {c}: {list(got)}"


def check_golden_layer(O):
    gm, ga, gp, gl = (load_golden(n) for n in
                      ("mlp_tiny.json", "mha_tiny.json", "predictor_tiny.json", "layer_tiny.json"))
    layer = dict(W1t=np.array(gm["W1t"]), W2t=np.array(gm["W2t"]), Wq=np.array(ga["Wq"]),
                 Wo=np.array(ga["Wo"]), K=np.array(ga["K"]), V=np.array(ga["V"]))
    nxt = dict(A_M=np.array(gp["A"]), B_M=np.array(gp["Bm"]), A_A=np.array(gl["next_A_A"]),
               B_A=np.array(gl["next_B_A"]), k_m=gl["next_k_m"], k_a=gl["next_k_a"], union=True)
    y = np.array(gm["y"])
    y_next, (sm, sa) = O.decode_layer(y, layer, gl["S_M"], gl["S_A"], nxt)
    assert_close(y_next, gl["y_next"], 1e-12, "layer y_next")
    assert list(sm) == gl["next_S_M"], f"next S_M {list(sm)}"
    assert list(sa) == gl["next_S_A"], f"next S_A {list(sa)}"


# --------------------------------------------------------------------------- #
# A1 predictor                                                                #
# --------------------------------------------------------------------------- #

def check_scores_associative(O):
    r = _rng(1)
    for (B, d, rk, N) in [(1, 8, 3, 11), (3, 16, 5, 7), (2, 33, 1, 40)]:
        y, A, Bm = r.standard_normal((B, d)), r.standard_normal((rk, d)), r.standard_normal((rk, N))
        s = O.predict_scores(y, A, Bm)
        # y (A B): the product of the two factors first, a different association.
        s_ref = y @ (A.T @ Bm)
        assert_close(s, s_ref, 1e-12, "scores y(AB)")


def check_scores_identity_factor(O):
    r = _rng(2)
    d, N = 6, 9
    y, Bm = r.standard_normal((2, d)), r.standard_normal((d, N))
    s = O.predict_scores(y, np.eye(d), Bm)      # A = I: s = y Bm
    ref = np.array([[sum(y[b, t] * Bm[t, j] for t in range(d)) for j in range(N)] for b in range(2)])
    assert_close(s, ref, 1e-13, "scores A=I")


def check_scores_bf16_widening(O):
    # bf16 bit patterns 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25, 0x0000 = 0.
    A = np.array([[0x3F80, 0xC000]], dtype=np.uint16)   # [r=1][d=2] = [1, -2]
    Bm = np.array([[0x3E80, 0x0000, 0xC000]], dtype=np.uint16)  # [1][3] = [0.25, 0, -2]
    s = O.predict_scores(np.array([[3.0, 1.0]]), A, Bm)  # z = 3 - 2 = 1
    assert_close(s, [[0.25, 0.0, -2.0]], 0.0, "bf16 widening")


# --------------------------------------------------------------------------- #
# A2 top-k and union                                                          #
# --------------------------------------------------------------------------- #

def _brute_topk(s, k):
    """The unique k-subset S with: i in S, j not in S => s_i > s_j or (s_i == s_j and i < j)."""
    N = len(s)
    k = max(0, min(k, N))
    found = []
    for S in itertools.combinations(range(N), k):
        Ss = set(S)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j)
                 for i in Ss for j in range(N) if j not in Ss)
        if ok:
            found.append(list(S))
    assert len(found) == 1, f"brute force found {len(found)} valid subsets"
    return found[0]


def check_topk_bruteforce(O):
    r = _rng(3)
    for trial in range(60):
        N = int(r.integers(1, 10))
        # few distinct values so that ties are common; include +-0
        vals = np.array([-1.0, -0.0, 0.0, 0.5, 2.0, 2.0, 3.0])
        s = r.choice(vals, size=N) if trial % 2 else r.standard_normal(N)
        for k in range(0, N + 2):
            got = list(O.topk_row(s, k))
            assert got == _brute_topk(list(s), k), f"trial {trial} s={s} k={k}: {got}"


def check_topk_lexsort(O):
    r = _rng(4)
    for N, k in [(1000, 100), (4096, 409), (257, 0), (300, 300), (50, 1)]:
        s = np.round(r.standard_normal(N) * 8) / 8       # 3 bits of fraction: many ties
        got = O.topk_row(s, k)
        ref = np.sort(np.lexsort((np.arange(N), -s))[:k])
        assert np.array_equal(got, ref), f"lexsort N={N} k={k}"


def check_topk_special(O):
    N = 37
    assert list(O.topk_row(np.full(N, 1.5), 5)) == list(range(5)), "constant scores"
    assert list(O.topk_row(np.arange(N, dtype=float), N)) == list(range(N)), "k = N"
    assert list(O.topk_row(np.arange(N, dtype=float), 0)) == [], "k = 0"
    s = np.arange(N, dtype=float)
    assert list(O.topk_row(s, 3)) == [N - 3, N - 2, N - 1], "increasing scores"
    r = _rng(5)
    s2 = r.standard_normal((1, 64))
    assert list(O.select_sets(s2, 7, True)) == list(O.topk_row(s2[0], 7)), "B=1 union"
    dup = np.repeat(s2, 3, axis=0)
    assert list(O.select_sets(dup, 7, True)) == list(O.topk_row(s2[0], 7)), "duplicated tokens"
    s3 = r.standard_normal((4, 64))
    per = O.select_sets(s3, 9, False)
    ref = np.unique(np.concatenate(per))
    assert list(O.select_sets(s3, 9, True)) == list(ref), "union = set union"
    for p in per:
        assert list(p) == sorted(p), "ascending"


# --------------------------------------------------------------------------- #
# A3 sparse MLP                                                               #
# --------------------------------------------------------------------------- #

def _mlp_data(seed, B=2, d=24, F=40):
    r = _rng(seed)
    return (r.standard_normal((B, d)), r.standard_normal((F, d)) * 0.3,
            r.standard_normal((F, d)) * 0.3)


def check_mlp_dense_library(O):
    y, W1t, W2t = _mlp_data(6)
    F, d = W1t.shape
    ffn = torch.nn.Sequential(torch.nn.Linear(d, F), torch.nn.ReLU(), torch.nn.Linear(F, d)).double()
    with torch.no_grad():
        ffn[0].weight.copy_(torch.from_numpy(W1t))     # nn.Linear weight is [out][in]
        ffn[0].bias.zero_()
        ffn[2].weight.copy_(torch.from_numpy(W2t.T.copy()))
        ffn[2].bias.zero_()
        ref = ffn(torch.from_numpy(y)).numpy()
    out = O.sparse_mlp(y, W1t, W2t, np.arange(F))
    assert_close(out, ref, 1e-12, "mlp S=all vs nn FFN")


def check_mlp_empty_and_additive(O):
    y, W1t, W2t = _mlp_data(7)
    F = W1t.shape[0]
    z = O.sparse_mlp(y, W1t, W2t, [])
    assert np.array_equal(z, np.zeros_like(y)), "empty set must give exact zero"
    r = _rng(8)
    perm = r.permutation(F)
    S1, S2 = perm[:13], perm[13:29]
    both = O.sparse_mlp(y, W1t, W2t, np.concatenate([S1, S2]))
    parts = O.sparse_mlp(y, W1t, W2t, S1) + O.sparse_mlp(y, W1t, W2t, S2)
    assert_close(both, parts, 1e-12, "mlp additivity")


def check_mlp_relu_support(O):
    y, W1t, W2t = _mlp_data(9, B=1)
    F = W1t.shape[0]
    a = y[0] @ W1t.T
    S_star = np.nonzero(a > 0)[0]
    assert 0 < len(S_star) < F
    assert_close(O.sparse_mlp(y, W1t, W2t, S_star), O.sparse_mlp(y, W1t, W2t, np.arange(F)),
                 1e-12, "ReLU support reproduces dense")
    S_neg = np.nonzero(a <= 0)[0]
    assert np.array_equal(O.sparse_mlp(y, W1t, W2t, S_neg), np.zeros_like(y)), "inactive set gives 0"


def check_mlp_loops(O):
    y, W1t, W2t = _mlp_data(10, B=2, d=5, F=7)
    S = [0, 2, 3, 6]
    ref = np.zeros_like(y)
    for b in range(2):
        for i in S:
            a = sum(y[b, j] * W1t[i, j] for j in range(5))
            h = a if a > 0 else 0.0
            for j in range(5):
                ref[b, j] += h * W2t[i, j]
    assert_close(O.sparse_mlp(y, W1t, W2t, S), ref, 1e-13, "mlp loops")


def check_mlp_set_order_irrelevant(O):
    y, W1t, W2t = _mlp_data(11)
    S = [5, 1, 30, 7]
    assert_close(O.sparse_mlp(y, W1t, W2t, S), O.sparse_mlp(y, W1t, W2t, sorted(S)), 1e-13,
                 "set order")


# GeLU (the page names it beside ReLU as sigma; section 2.3 under Eq. (1)).
# Standard normal CDF values as tabulated (e.g. Abramowitz & Stegun, table 26.1):
# GeLU(x) = x Phi(x).
PHI_TABLE = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429, 2.0: 0.9772498680518208,
             -1.0: 0.15865525393145707, -2.5: 0.006209665325776159}


def check_gelu_values(O):
    for x, phi in PHI_TABLE.items():
        got = float(O.gelu(np.array([x]))[0])
        assert abs(got - x * phi) <= 1e-15 * max(1.0, abs(x)), f"gelu({x}) = {got} vs {x * phi}"
    assert float(O.gelu(np.array([0.0]))[0]) == 0.0, "gelu(0) must be 0"
    big = float(O.gelu(np.array([40.0]))[0])
    assert big == 40.0, "gelu(x) = x for large x"


def check_mlp_gelu_dense_library(O):
    y, W1t, W2t = _mlp_data(16)
    F, d = W1t.shape
    ffn = torch.nn.Sequential(torch.nn.Linear(d, F), torch.nn.GELU(approximate="none"),
                              torch.nn.Linear(F, d)).double()
    with torch.no_grad():
        ffn[0].weight.copy_(torch.from_numpy(W1t))
        ffn[0].bias.zero_()
        ffn[2].weight.copy_(torch.from_numpy(W2t.T.copy()))
        ffn[2].bias.zero_()
        ref = ffn(torch.from_numpy(y)).numpy()
    out = O.sparse_mlp(y, W1t, W2t, np.arange(F), "gelu")
    assert_close(out, ref, 1e-12, "gelu mlp S=all vs nn FFN")


def check_mlp_gelu_loops_and_additive(O):
    import math
    y, W1t, W2t = _mlp_data(17, B=2, d=5, F=7)
    S = [1, 2, 4, 6]
    ref = np.zeros_like(y)
    for b in range(2):
        for i in S:
            a = sum(y[b, j] * W1t[i, j] for j in range(5))
            h = a * 0.5 * (1.0 + math.erf(a / math.sqrt(2.0)))
            for j in range(5):
                ref[b, j] += h * W2t[i, j]
    assert_close(O.sparse_mlp(y, W1t, W2t, S, "gelu"), ref, 1e-13, "gelu mlp loops")
    both = O.sparse_mlp(y, W1t, W2t, S, "gelu")
    parts = O.sparse_mlp(y, W1t, W2t, S[:2], "gelu") + O.sparse_mlp(y, W1t, W2t, S[2:], "gelu")
    assert_close(both, parts, 1e-13, "gelu mlp additivity")
    assert np.array_equal(O.sparse_mlp(y, W1t, W2t, [], "gelu"), np.zeros_like(y))


def check_layer_gelu(O):
    r = _rng(18)
    B, d, F, h, dh, n = 2, 8, 12, 2, 4, 3
    layer = dict(W1t=r.standard_normal((F, d)), W2t=r.standard_normal((F, d)),
                 Wq=r.standard_normal((h, dh, d)), Wo=r.standard_normal((h, dh, d)),
                 K=r.standard_normal((B, h, n, dh)), V=r.standard_normal((B, h, n, dh)), act="gelu")
    y = r.standard_normal((B, d))
    S_M, S_A = [0, 3, 5, 11], [1]
    got, _ = O.decode_layer(y, layer, S_M, S_A, None)
    want = y + O.sparse_mlp(y, layer["W1t"], layer["W2t"], S_M, "gelu") + \
        O.sparse_mha(y, layer["Wq"], layer["Wo"], layer["K"], layer["V"], S_A)
    assert_close(got, want, 1e-13, "layer with gelu")
    relu_out, _ = O.decode_layer(y, dict(layer, act="relu"), S_M, S_A, None)
    assert rel_diff(got, relu_out) > 1e-3, "layer ignores its activation"


def rel_diff(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) / max(1e-300, float(np.max(np.abs(b))))


# Weight-only fp8 (E4M3 codes with one scale per row).  Independent references:
# torch's float8_e4m3fn decoder for all 256 codes, and values of the OCP format
# worked out by hand from its definition (bias 7, 3 mantissa bits, subnormals at
# exponent field 0, S.1111.111 = NaN, largest finite 448).
E4M3_HAND = {0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x3C: 1.5, 0xB0: -0.5, 0x7E: 448.0, 0xFE: -448.0, 0x77: 240.0}


def _torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def check_e4m3_decode(O):
    got = O.decode_e4m3(np.arange(256, dtype=np.uint8))
    ref = _torch_e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "E4M3 NaN codes"
    assert np.array_equal(got[~nan], ref[~nan]), "E4M3 decode vs torch float8_e4m3fn"
    for c, v in E4M3_HAND.items():
        g = float(O.decode_e4m3(np.array([c], dtype=np.uint8))[0])
        assert g == v and np.signbit(g) == np.signbit(v), f"E4M3 code {c:#04x}: {g} vs {v}"
    assert np.isnan(O.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def _fp8_rows(seed, shape):
    """Random fp8 row storage (no NaN codes) and its dense value, built row by row
    from torch's decoder: (codes, scales, dense float64)."""
    r = _rng(seed)
    codes = r.integers(0, 256, size=shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    scales = r.uniform(0.001, 0.01, size=shape[:-1])
    table = _torch_e4m3_table()
    dense = np.zeros(shape)
    for ix in np.ndindex(*shape[:-1]):
        dense[ix] = scales[ix] * table[codes[ix]]
    return codes, scales, dense


def check_fp8_rows_mlp_mha(O):
    y = _rng(20).standard_normal((2, 32))
    c1, s1, W1 = _fp8_rows(21, (40, 32))
    c2, s2, W2 = _fp8_rows(22, (40, 32))
    S = [0, 5, 17, 39]
    assert_close(O.sparse_mlp(y, O.Fp8Rows(c1, s1), O.Fp8Rows(c2, s2), S),
                 O.sparse_mlp(y, W1, W2, S), 1e-13, "fp8 rows mlp vs dense dequantized")
    cq, sq, Wq = _fp8_rows(23, (3, 4, 32))
    co, so, Wo = _fp8_rows(24, (3, 4, 32))
    r = _rng(25)
    K, V = r.standard_normal((2, 3, 5, 4)), r.standard_normal((2, 3, 5, 4))
    assert_close(O.sparse_mha(y, O.Fp8Rows(cq, sq), O.Fp8Rows(co, so), K, V, [0, 2]),
                 O.sparse_mha(y, Wq, Wo, K, V, [0, 2]), 1e-13, "fp8 rows mha vs dense dequantized")


# --------------------------------------------------------------------------- #
# A4 sparse MHA                                                               #
# --------------------------------------------------------------------------- #

def _mha_data(seed, B=2, d=16, h=3, dh=4, n=7):
    r = _rng(seed)
    return (r.standard_normal((B, d)), r.standard_normal((h, dh, d)) * 0.3,
            r.standard_normal((h, dh, d)) * 0.3, r.standard_normal((B, h, n, dh)),
            r.standard_normal((B, h, n, dh)))


def check_mha_dense_library(O):
    for scale in (1.0, 0.5):
        y, Wq, Wo, K, V = _mha_data(12)
        B, d = y.shape
        h, dh, _ = Wq.shape
        yt = torch.from_numpy(y)
        q = torch.einsum("bd,icd->bic", yt, torch.from_numpy(Wq))      # [B][h][dh]
        o = torch.nn.functional.scaled_dot_product_attention(
            q.unsqueeze(2), torch.from_numpy(K), torch.from_numpy(V), scale=scale)  # [B][h][1][dh]
        Z = o.squeeze(2).reshape(B, h * dh)          # concatenate heads in order
        ref = (Z @ torch.from_numpy(Wo).reshape(h * dh, d)).numpy()
        out = O.sparse_mha(y, Wq, Wo, K, V, np.arange(h), scale)
        assert_close(out, ref, 1e-12, f"mha S=all vs sdpa scale={scale}")


def check_mha_empty_and_additive(O):
    y, Wq, Wo, K, V = _mha_data(13, h=5)
    assert np.array_equal(O.sparse_mha(y, Wq, Wo, K, V, []), np.zeros_like(y)), "empty heads"
    both = O.sparse_mha(y, Wq, Wo, K, V, [0, 2, 4])
    parts = O.sparse_mha(y, Wq, Wo, K, V, [0, 4]) + O.sparse_mha(y, Wq, Wo, K, V, [2])
    assert_close(both, parts, 1e-12, "mha additivity")


def check_head_closed_forms(O):
    r = _rng(14)
    d, dh = 8, 4
    y, WQ = r.standard_normal(d), r.standard_normal((d, dh))
    V1 = r.standard_normal((1, dh))
    assert_close(O.head_output(y, WQ, r.standard_normal((1, dh)), V1), V1[0], 1e-15, "n=1")
    Vn = r.standard_normal((6, dh))
    Keq = np.tile(r.standard_normal((1, dh)), (6, 1))
    assert_close(O.head_output(y, WQ, Keq, Vn), Vn.mean(axis=0), 1e-13, "equal keys -> mean")
    q = y @ WQ
    Kdom = r.standard_normal((6, dh)) * 0.01
    Kdom[3] = 1e3 * q / np.linalg.norm(q)          # logit of key 3 far above the rest
    assert_close(O.head_output(y, WQ, Kdom, Vn), Vn[3], 1e-12, "dominant key")
    # scale: logits scale linearly
    K = r.standard_normal((5, dh))
    assert_close(O.head_output(y, WQ, K, Vn[:5], 2.0), O.head_output(y, 2.0 * WQ, K, Vn[:5], 1.0),
                 1e-12, "scale folds into W^Q")


def check_head_mean_shift(O):
    """Deja Vu page, section 3.2: K_i(x_j, y) = exp(y W^Q (W^K)^T x_j),
    m_i(y) = sum_j K_i(x_j, y) x_j / sum_j K_i(x_j, y) and H_i(y) = m_i(y) W^V."""
    r = _rng(15)
    n, d, dh = 6, 10, 3
    X = r.standard_normal((n, d)) * 0.5
    WQ, WK, WV = (r.standard_normal((d, dh)) * 0.5 for _ in range(3))
    y = r.standard_normal(d)
    sim = [np.exp(sum(sum(y[a] * WQ[a, c] for a in range(d)) * sum(WK[e, c] * X[j, e] for e in range(d))
                      for c in range(dh))) for j in range(n)]
    m = sum(sim[j] * X[j] for j in range(n)) / sum(sim)
    ref = m @ WV
    got = O.head_output(y, WQ, X @ WK, X @ WV)
    assert_close(got, ref, 1e-12, "mean-shift form")


# --------------------------------------------------------------------------- #
# A5 layer                                                                    #
# --------------------------------------------------------------------------- #

def check_layer_composition(O):
    y, Wq, Wo, K, V = _mha_data(16, B=2, d=12, h=4, dh=3, n=5)
    r = _rng(17)
    F = 20
    W1t, W2t = r.standard_normal((F, 12)), r.standard_normal((F, 12))
    layer = dict(W1t=W1t, W2t=W2t, Wq=Wq, Wo=Wo, K=K, V=V)
    nxt = dict(A_M=r.standard_normal((3, 12)), B_M=r.standard_normal((3, F)),
               A_A=r.standard_normal((3, 12)), B_A=r.standard_normal((3, 4)),
               k_m=6, k_a=2, union=True)
    S_M, S_A = [1, 4, 9, 15], [0, 3]
    y_next, (sm, sa) = O.decode_layer(y, layer, S_M, S_A, nxt)
    ref = y + O.sparse_mlp(y, W1t, W2t, S_M) + O.sparse_mha(y, Wq, Wo, K, V, S_A)
    assert_close(y_next, ref, 1e-13, "layer = y + mlp + mha")
    sm_ref = O.select_sets(O.predict_scores(y, nxt["A_M"], nxt["B_M"]), 6, True)
    assert list(sm) == list(sm_ref), "next sets from the layer input"
    _, none = O.decode_layer(y, layer, S_M, S_A, None)
    assert none is None


def check_stack_lookahead(O):
    r = _rng(18)
    d, F, h, dh, n, B = 6, 10, 3, 2, 4, 2
    def mk():
        return dict(W1t=r.standard_normal((F, d)), W2t=r.standard_normal((F, d)),
                    Wq=r.standard_normal((h, dh, d)), Wo=r.standard_normal((h, dh, d)),
                    K=r.standard_normal((B, h, n, dh)), V=r.standard_normal((B, h, n, dh)),
                    A_M=r.standard_normal((2, d)), B_M=r.standard_normal((2, F)),
                    A_A=r.standard_normal((2, d)), B_A=r.standard_normal((2, h)),
                    k_m=3, k_a=1, union=True)
    layers = [mk() for _ in range(3)]
    y0 = r.standard_normal((B, d))
    yL, used = O.decode_stack(y0, layers)
    # unrolled by hand: layer 0 predicts its own sets from y0; layer l+1 from y_l
    def sets(y, L):
        return (O.select_sets(O.predict_scores(y, L["A_M"], L["B_M"]).astype(np.float32), 3, True),
                O.select_sets(O.predict_scores(y, L["A_A"], L["B_A"]).astype(np.float32), 1, True))
    y, expect = y0, []
    s = sets(y0, layers[0])
    for l in range(3):
        expect.append(s)
        nxt = sets(y, layers[l + 1]) if l + 1 < 3 else None
        y = y + O.sparse_mlp(y, layers[l]["W1t"], layers[l]["W2t"], s[0]) + \
            O.sparse_mha(y, layers[l]["Wq"], layers[l]["Wo"], layers[l]["K"], layers[l]["V"], s[1])
        s = nxt
    assert_close(yL, y, 1e-12, "stack output")
    for (a0, a1), (b0, b1) in zip(used, expect):
        assert list(a0) == list(b0) and list(a1) == list(b1), "stack sets"


# --------------------------------------------------------------------------- #
# the full decode step: the current token's k and v join the cache            #
# --------------------------------------------------------------------------- #

def check_round_bf16(O):
    """Storage rounding of appended rows: nearest bf16, ties to even, rounded once
    from float64.  Against torch's float32 -> bfloat16 cast where the value is a
    float32 (one rounding either way), and hand-worked bit patterns."""
    r = _rng(30)
    x = r.standard_normal(20000) * np.exp2(r.integers(-30, 30, 20000).astype(np.float64))
    x = np.concatenate([x, np.exp2(np.arange(-133, -120, dtype=np.float64)) * 1.37])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.round_bf16(x32.astype(np.float64))
    assert got.dtype == np.uint16 and np.array_equal(got, ref), "bf16 rounding vs torch"
    hand = [(1.0, 0x3F80), (1 + 2.0 ** -8, 0x3F80),         # tie, even neighbour below
            (1 + 3 * 2.0 ** -8, 0x3F82),                      # tie, even neighbour above
            (1 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),             # just above the tie: one rounding
            (-2.5, 0xC020), (-0.0, 0x8000), (0.0, 0x0000),
            (2.0 ** -130, 0x0008),                            # bf16 subnormal
            (255.5, 0x4380), (257.0, 0x4380), (259.0, 0x4382)]   # 8 significant bits
    for v, bits in hand:
        assert int(O.round_bf16(np.array([v]))[0]) == bits, f"round_bf16({v!r})"


def _append_data(seed, B=2, d=12, h=4, dh=3, n=6, F=16):
    r = _rng(seed)
    X = r.standard_normal((B, n + 1, d))          # each token's sequence; row n is the current token
    W = {k: r.standard_normal((h, dh, d)) * 0.4 for k in ("Wq", "Wk", "Wv", "Wo")}
    W["W1t"], W["W2t"] = r.standard_normal((F, d)), r.standard_normal((F, d))
    return X, W


def check_append_equals_recompute(O):
    """KV-cache blog page, figure (b): caching the keys and values and appending the
    current token's gives what attention over the whole sequence gives.  Reference:
    the last query of causal scaled_dot_product_attention over all n + 1 tokens,
    projected by W^O of the selected heads; the appended rows are the last rows of
    X W^K and X W^V for every head."""
    for scale in (1.0, 0.7):
        X, W = _append_data(31)
        B, n1, d = X.shape
        n = n1 - 1
        h, dh, _ = W["Wq"].shape
        Xt = torch.from_numpy(X)
        proj = {k: torch.einsum("bnd,icd->bin c".replace(" ", ""), Xt, torch.from_numpy(W[k]))
                for k in ("Wq", "Wk", "Wv")}                       # [B][h][n+1][dh]
        cap = n + 3
        K = np.full((B, h, cap, dh), 7.0)
        V = np.full((B, h, cap, dh), -7.0)
        K[:, :, :n] = proj["Wk"][:, :, :n].numpy()
        V[:, :, :n] = proj["Wv"][:, :, :n].numpy()
        K0, V0 = K.copy(), V.copy()
        S_A = [0, 2, 3]
        layer = dict(W1t=W["W1t"], W2t=W["W2t"], Wq=W["Wq"], Wo=W["Wo"], Wk=W["Wk"],
                     Wv=W["Wv"], K=K, V=V)
        y = X[:, n]
        y_next, _, (k_row, v_row) = O.decode_layer_append(y, layer, [], S_A, None, n, scale)
        assert np.array_equal(K, K0) and np.array_equal(V, V0), "inputs modified"
        o = torch.nn.functional.scaled_dot_product_attention(
            proj["Wq"], proj["Wk"], proj["Wv"], is_causal=True, scale=scale)[:, :, n]   # [B][h][dh]
        ref = sum(o[:, i] @ torch.from_numpy(W["Wo"][i]) for i in S_A).numpy()
        assert_close(y_next - y, ref, 1e-12, f"append = attention over the sequence, scale {scale}")
        assert_close(k_row, proj["Wk"][:, :, n].numpy(), 1e-13, "appended keys, every head")
        assert_close(v_row, proj["Wv"][:, :, n].numpy(), 1e-13, "appended values, every head")
        try:
            O.decode_layer_append(y, layer, [], S_A, None, cap, scale)
        except ValueError:
            pass
        else:
            raise AssertionError("a row outside the cache must be refused")


def check_append_stored_row_attended(O):
    """With a bf16 cache the stored (rounded) row is the one attended: the step's
    output is Eq. (2) over the widened cache rows 0..n-1 plus the returned row,
    computed here with scaled_dot_product_attention; and an empty cache (n = 0)
    gives each selected head exactly its stored value row."""
    X, W = _append_data(32, n=5)
    B, n1, d = X.shape
    n = n1 - 1
    h, dh, _ = W["Wq"].shape
    r = _rng(33)
    Kb = torch.from_numpy(r.standard_normal((B, h, n + 2, dh))).to(torch.bfloat16)
    Vb = torch.from_numpy(r.standard_normal((B, h, n + 2, dh))).to(torch.bfloat16)
    K = Kb.view(torch.int16).numpy().view(np.uint16)
    V = Vb.view(torch.int16).numpy().view(np.uint16)
    layer = dict(W1t=W["W1t"], W2t=W["W2t"], Wq=W["Wq"], Wo=W["Wo"], Wk=W["Wk"], Wv=W["Wv"],
                 K=K, V=V)
    y = X[:, n]
    S_A = [1, 3]
    y_next, _, (k_row, v_row) = O.decode_layer_append(y, layer, [], S_A, None, n)
    assert k_row.dtype == np.uint16 and v_row.dtype == np.uint16, "rows stored as bf16"
    wid = lambda a: torch.from_numpy(a.astype(np.uint32) << 16).view(torch.float32).double()  # noqa: E731
    Kc = torch.cat([Kb[:, :, :n].double(), wid(k_row).unsqueeze(2)], dim=2)
    Vc = torch.cat([Vb[:, :, :n].double(), wid(v_row).unsqueeze(2)], dim=2)
    q = torch.einsum("bd,icd->bic", torch.from_numpy(y), torch.from_numpy(W["Wq"]))
    o = torch.nn.functional.scaled_dot_product_attention(q.unsqueeze(2), Kc, Vc, scale=1.0).squeeze(2)
    ref = sum(o[:, i] @ torch.from_numpy(W["Wo"][i]) for i in S_A).numpy()
    assert_close(y_next - y, ref, 1e-12, "bf16 cache: stored row attended")
    v_exact = np.einsum("bd,icd->bic", y, W["Wv"])
    assert np.max(np.abs(wid(v_row).numpy() - v_exact) / np.maximum(np.abs(v_exact), 1e-30)) \
        <= 2.0 ** -8, "stored values within half a bf16 ulp (2^-8 relative)"
    # empty cache: softmax over one key is 1, H_i = v_i
    y0, _, (_, v0) = O.decode_layer_append(y, layer, [], S_A, None, 0)
    ref0 = sum(wid(v0)[:, i].numpy() @ W["Wo"][i] for i in S_A)
    assert_close(y0 - y, ref0, 1e-13, "n = 0: each head returns its own value")


def check_append_every_head_two_steps(O):
    """Why the append stores every head's row (the KV-cache blog page, figure (b), with
    Eq. (2), whose X holds every previous token for every head): over two steps whose
    head sets differ, the second step's heads, skipped by the first, still attend over
    the first step's token.  Reference: causal scaled_dot_product_attention over all
    n + 2 tokens.  Storing only the first step's selected heads (the alternative reading,
    which at OPT-175B would read 2 x 19 x 128 rows of 24 KiB, 119.5 MB, instead of
    2 x 96 x 128, 604 MB) leaves those heads without the token, and the second step's
    output then departs from the reference."""
    X, W = _append_data(34, n=7)                         # 8 tokens: n = 6 cached, two steps
    B, n2, d = X.shape
    n = n2 - 2
    h, dh, _ = W["Wq"].shape
    Xt = torch.from_numpy(X)
    proj = {k: torch.einsum("bnd,icd->binc", Xt, torch.from_numpy(W[k]))
            for k in ("Wq", "Wk", "Wv")}                 # [B][h][n+2][dh]
    cap = n + 3
    K = np.full((B, h, cap, dh), 7.0)
    V = np.full((B, h, cap, dh), -7.0)
    K[:, :, :n] = proj["Wk"][:, :, :n].numpy()
    V[:, :, :n] = proj["Wv"][:, :, :n].numpy()
    S1, S2 = [0, 2], [1, 3]                              # the second step's heads skipped the first
    base = dict(W1t=W["W1t"], W2t=W["W2t"], Wq=W["Wq"], Wo=W["Wo"], Wk=W["Wk"], Wv=W["Wv"])
    _, _, (k1, v1) = O.decode_layer_append(X[:, n], dict(base, K=K, V=V), [], S1, None, n)
    o = torch.nn.functional.scaled_dot_product_attention(
        proj["Wq"], proj["Wk"], proj["Wv"], is_causal=True, scale=1.0)[:, :, n + 1]   # [B][h][dh]
    ref = sum(o[:, i] @ torch.from_numpy(W["Wo"][i]) for i in S2).numpy()
    # every head's row stored (the reading built): the second step matches the sequence
    Ka, Va = K.copy(), V.copy()
    Ka[:, :, n], Va[:, :, n] = k1, v1
    y2, _, _ = O.decode_layer_append(X[:, n + 1], dict(base, K=Ka, V=Va), [], S2, None, n + 1)
    assert_close(y2 - X[:, n + 1], ref, 1e-12, "every head stored: second step = attention over the sequence")
    # only the first step's heads stored: heads 1 and 3 miss token n
    Ks, Vs = K.copy(), V.copy()
    Ks[:, S1, n], Vs[:, S1, n] = k1[:, S1], v1[:, S1]
    y2s, _, _ = O.decode_layer_append(X[:, n + 1], dict(base, K=Ks, V=Vs), [], S2, None, n + 1)
    gap = np.max(np.abs((y2s - X[:, n + 1]) - ref)) / np.max(np.abs(ref))
    assert gap > 1e-3, f"storing the selected heads only should change the output (gap {gap:.2e})"


ALL_CHECKS = [
    check_golden_mlp, check_golden_mha, check_golden_predictor, check_golden_layer,
    check_scores_associative, check_scores_identity_factor, check_scores_bf16_widening,
    check_topk_bruteforce, check_topk_lexsort, check_topk_special,
    check_mlp_dense_library, check_mlp_empty_and_additive, check_mlp_relu_support,
    check_mlp_loops, check_mlp_set_order_irrelevant,
    check_gelu_values, check_mlp_gelu_dense_library, check_mlp_gelu_loops_and_additive,
    check_layer_gelu, check_e4m3_decode, check_fp8_rows_mlp_mha,
    check_mha_dense_library, check_mha_empty_and_additive, check_head_closed_forms,
    check_head_mean_shift, check_layer_composition, check_stack_lookahead,
    check_round_bf16, check_append_equals_recompute, check_append_stored_row_attended,
    check_append_every_head_two_steps,
]
