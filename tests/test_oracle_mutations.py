"""Plant a plausible mistake in the oracle (on the CPU, never on the GPU) and
require that at least one pin fails.  This shows that the pins would catch a
dropped term, a wrong sign or index, or a transposed operand."""
import types

import numpy as np
import pytest
import torch

import pins
from oracle import dv_oracle as O


def _mutant(**overrides):
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update({k: v for k, v in O.__dict__.items() if k not in ("__name__", "__spec__")})
    m.__dict__.update(overrides)
    # functions close over the real module's globals; rebind them to the mutant
    for name, fn in list(m.__dict__.items()):
        if isinstance(fn, types.FunctionType) and name not in overrides:
            m.__dict__[name] = types.FunctionType(fn.__code__, m.__dict__, fn.__name__,
                                                  fn.__defaults__, fn.__closure__)
    return m


def _mlp_no_relu(y, W1t, W2t, S_M, act="relu"):
    y = O.widen(y); S = O.as_set(S_M)
    return (y @ O.rows(W1t, S).T) @ O.rows(W2t, S)


def _mlp_swapped(y, W1t, W2t, S_M, act="relu"):
    y = O.widen(y); S = O.as_set(S_M)
    return O.activation(act)(y @ O.rows(W2t, S).T) @ O.rows(W1t, S)


def _mlp_dropped_last(y, W1t, W2t, S_M, act="relu"):
    S = O.as_set(S_M)
    return O.sparse_mlp(y, W1t, W2t, S[:-1], act) if len(S) > 1 else O.sparse_mlp(y, W1t, W2t, S, act)


def _gelu_tanh(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def _gelu_no_half(x):
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return x * (1.0 + erf(x / np.sqrt(2.0)))


def _gelu_no_sqrt2(x):
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x))


def _mlp_act_ignored(y, W1t, W2t, S_M, act="relu"):
    return O.sparse_mlp(y, W1t, W2t, S_M, "relu")


def _head_div_n(y_b, WQ_i, K_bi, V_bi, scale=1.0):
    q = y_b @ WQ_i
    t = scale * (q @ K_bi.T)
    e = np.exp(t - t.max())
    return (e @ V_bi) / len(t)


def _head_values_from_keys(y_b, WQ_i, K_bi, V_bi, scale=1.0):
    q = y_b @ WQ_i
    t = scale * (q @ K_bi.T)
    e = np.exp(t - t.max())
    return (e @ K_bi) / e.sum()


def _head_no_scale(y_b, WQ_i, K_bi, V_bi, scale=1.0):
    return O.head_output(y_b, WQ_i, K_bi, V_bi, 1.0)


def _head_neg_logits(y_b, WQ_i, K_bi, V_bi, scale=1.0):
    q = y_b @ WQ_i
    t = -scale * (q @ K_bi.T)
    e = np.exp(t - t.max())
    return (e @ V_bi) / e.sum()


def _mha_wo_transposed(y, Wq, Wo, K, V, S_A, scale=1.0):
    y = O.widen(y)
    out = np.zeros_like(y)
    for i in O.as_set(S_A):
        WQ_i = O.widen(np.asarray(Wq)[i]).T
        WO_i = O.widen(np.asarray(Wq)[i])          # wrong tensor
        for b in range(y.shape[0]):
            out[b] += O.head_output(y[b], WQ_i, O.widen(np.asarray(K)[b, i]),
                                    O.widen(np.asarray(V)[b, i]), scale) @ WO_i
    return out


def _topk_high_index_ties(s, k):
    s = np.asarray(s, dtype=np.float64)
    N = len(s); k = max(0, min(int(k), N))
    order = sorted(range(N), key=lambda j: (-s[j], -j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def _topk_smallest(s, k):
    s = np.asarray(s, dtype=np.float64)
    N = len(s); k = max(0, min(int(k), N))
    order = sorted(range(N), key=lambda j: (s[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def _topk_unsorted(s, k):
    s = np.asarray(s, dtype=np.float64)
    N = len(s); k = max(0, min(int(k), N))
    return np.array(sorted(range(N), key=lambda j: (-s[j], j))[:k], dtype=np.int64)


def _topk_off_by_one(s, k):
    return O.topk_row(s, max(0, k - 1)) if k > 1 else O.topk_row(s, k)


def _scores_no_second_factor(y, A, Bm):
    return O.widen(y) @ O.widen(A).T @ np.ones((np.asarray(A).shape[0], np.asarray(Bm).shape[1]))


def _scores_transposed_A(y, A, Bm):
    y = O.widen(y); A = O.widen(A)
    z = (A @ y.T).T if A.shape[0] == A.shape[1] else y @ A.T
    return (y @ A) @ O.widen(Bm) if A.shape[0] == A.shape[1] else z @ O.widen(Bm)


def _layer_predict_from_output(y, layer, S_M, S_A, next_layer, scale=1.0):
    y_next, _ = O.decode_layer(y, layer, S_M, S_A, None, scale)
    sets = None
    if next_layer is not None:
        sets = (O.predict_and_select(y_next, next_layer["A_M"], next_layer["B_M"],
                                     next_layer["k_m"], next_layer["union"]),
                O.predict_and_select(y_next, next_layer["A_A"], next_layer["B_A"],
                                     next_layer["k_a"], next_layer["union"]))
    return y_next, sets


def _layer_no_residual(y, layer, S_M, S_A, next_layer, scale=1.0):
    y_next, sets = O.decode_layer(y, layer, S_M, S_A, next_layer, scale)
    return y_next - O.widen(y), sets


def _layer_no_mha(y, layer, S_M, S_A, next_layer, scale=1.0):
    return O.decode_layer(y, layer, S_M, [], next_layer, scale)


def _union_as_intersection(scores, k, union):
    per = [O.topk_row(r, k) for r in np.asarray(scores)]
    if not union:
        return per
    out = per[0]
    for p in per[1:]:
        out = np.intersect1d(out, p)
    return out


def _widen_wrong_shift(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _e4m3_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, sign * val)


def _e4m3_no_subnormals(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, sign * val)


def _widen_fp8_no_scale(a):
    if isinstance(a, O.Fp8Rows):
        return O.decode_e4m3(a.codes)
    return O.widen(a)


def _append_ignores_current(y, layer, S_M, S_A, next_layer, n, scale=1.0):
    k, v = O.kv_for_token(y, layer["Wk"], layer["Wv"])
    K, V = np.asarray(layer["K"]), np.asarray(layer["V"])
    lay = dict(layer, K=K[:, :, :n], V=V[:, :, :n])
    y_next, sets = O.decode_layer(y, lay, S_M, S_A, next_layer, scale) if n > 0 else \
        (O.widen(y) + O.sparse_mlp(y, layer["W1t"], layer["W2t"], S_M), None)
    return y_next, sets, (O.store_as(k, K), O.store_as(v, V))


def _append_overwrites_last(y, layer, S_M, S_A, next_layer, n, scale=1.0):
    return O.decode_layer_append(y, layer, S_M, S_A, next_layer, max(n - 1, 0), scale)


def _kv_swapped(y, Wk, Wv):
    k, v = _real_kv(y, Wk, Wv)
    return v, k


def _kv_selected_only(y, layer, S_M, S_A, next_layer, n, scale=1.0):
    y_next, sets, (k, v) = O.decode_layer_append(y, layer, S_M, S_A, next_layer, n, scale)
    keep = np.zeros(k.shape[1], dtype=bool)
    keep[O.as_set(S_A)] = True
    k, v = k.copy(), v.copy()
    k[:, ~keep] = 0
    v[:, ~keep] = 0
    return y_next, sets, (k, v)


def _append_attends_unrounded(y, layer, S_M, S_A, next_layer, n, scale=1.0):
    k, v = O.kv_for_token(y, layer["Wk"], layer["Wv"])
    K, V = np.asarray(layer["K"]), np.asarray(layer["V"])
    K1 = np.concatenate([O.widen(K[:, :, :n]), k[:, :, None]], axis=2)
    V1 = np.concatenate([O.widen(V[:, :, :n]), v[:, :, None]], axis=2)
    y_next, sets = O.decode_layer(y, dict(layer, K=K1, V=V1), S_M, S_A, next_layer, scale)
    return y_next, sets, (O.store_as(k, K), O.store_as(v, V))


def _bf16_truncate(x):
    v = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_via_f32(x):
    v = torch.from_numpy(np.asarray(x, dtype=np.float64).astype(np.float32)).to(torch.bfloat16)
    return v.view(torch.int16).numpy().view(np.uint16)


_real_kv = O.kv_for_token

MUTANTS = {
    "mlp without ReLU": dict(sparse_mlp=_mlp_no_relu),
    "mlp W1/W2 swapped": dict(sparse_mlp=_mlp_swapped),
    "mlp drops a neuron": dict(sparse_mlp=_mlp_dropped_last),
    "relu as identity": dict(relu=lambda x: x),
    "relu keeps negative part": dict(relu=lambda x: np.minimum(x, 0.0)),
    "gelu tanh approximation": dict(gelu=_gelu_tanh),
    "gelu without the half": dict(gelu=_gelu_no_half),
    "gelu erf without sqrt 2": dict(gelu=_gelu_no_sqrt2),
    "mlp ignores the activation": dict(sparse_mlp=_mlp_act_ignored),
    "head divides by n": dict(head_output=_head_div_n),
    "head uses keys as values": dict(head_output=_head_values_from_keys),
    "head ignores scale": dict(head_output=_head_no_scale),
    "head negated logits": dict(head_output=_head_neg_logits),
    "mha uses W^Q as W^O": dict(sparse_mha=_mha_wo_transposed),
    "top-k ties to higher index": dict(topk_row=_topk_high_index_ties),
    "top-k smallest": dict(topk_row=_topk_smallest),
    "top-k not ascending": dict(topk_row=_topk_unsorted),
    "top-k off by one": dict(topk_row=_topk_off_by_one),
    "scores drop second factor": dict(predict_scores=_scores_no_second_factor),
    "scores transposed factor": dict(predict_scores=_scores_transposed_A),
    "union as intersection": dict(select_sets=_union_as_intersection),
    "bf16 widening wrong": dict(widen=_widen_wrong_shift),
    "e4m3 exponent bias 8": dict(decode_e4m3=_e4m3_bias8),
    "e4m3 without subnormals": dict(decode_e4m3=_e4m3_no_subnormals),
    "fp8 rows ignore the scale": dict(widen=_widen_fp8_no_scale),
    "layer predicts from output": dict(decode_layer=_layer_predict_from_output),
    "layer drops residual": dict(decode_layer=_layer_no_residual),
    "layer drops attention": dict(decode_layer=_layer_no_mha),
    "append ignores the current token": dict(decode_layer_append=_append_ignores_current),
    "append overwrites the last cached row": dict(decode_layer_append=_append_overwrites_last),
    "append keys and values swapped": dict(kv_for_token=_kv_swapped),
    "append stores selected heads only": dict(decode_layer_append=_kv_selected_only),
    "append attends the unrounded row": dict(decode_layer_append=_append_attends_unrounded),
    "bf16 store truncates": dict(round_bf16=_bf16_truncate),
    "bf16 store rounds twice": dict(round_bf16=_bf16_via_f32),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    m = _mutant(**MUTANTS[name])
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check(m)
        except (AssertionError, ValueError, IndexError) as e:
            failures.append((check.__name__, str(e)[:80]))
    assert failures, f"no pin caught the planted mistake '{name}'"
