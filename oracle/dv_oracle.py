"""CPU oracle for the Deja Vu sparse decode step (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never calls it and shares no code with it.

Everything here is plain and slow on purpose: float64 NumPy, one library
primitive per step (a matrix product, a sort), no blocking, fusion or reordering
beyond what the definitions state.  Sources, cited by page title and section:

* "Deja Vu: contextual sparsity for efficient LLMs at inference time"
  (Chinese translation), section 2.3, Eq. (1): the sparse MLP
  MLP_{S_M}(y) = sigma(y W1_{S_M}) (W2_{S_M})^T with S_M a subset of [4d] and
  W1_i, W2_i the d-long columns of neuron i.
* same page, section 2.3, Eq. (2): the sparse MHA
  MHA_{S_A}(y) = sum_{i in S_A} H_i(y) W_i^O,
  H_i(y) = D_i(y)^{-1} exp(y W_i^Q (W_i^K)^T X^T) X W_i^V,
  D_i(y) = exp(y W_i^Q (W_i^K)^T X^T) 1_n.
* same page, section 1 (contribution list naming sections 4.1-4.3, whose text is
  not on the page): a low-overhead learned predictor that, from a layer's input,
  picks the heads and neurons of the next layer, run asynchronously one layer ahead.
  The predictor's form is not given there; this oracle takes the plainest reading,
  a two-factor low-rank map s = (y A) B with no bias and no nonlinearity (a
  monotone squashing would not change a top-k), and deterministic top-k with the
  lower index winning ties.

Readings where the pages are silent (each is listed in the design notes):
  sigma is ReLU unless GeLU is asked for (the page names both, section 2.3 under
  Eq. (1)); GeLU is the exact x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, Phi the
  standard normal CDF (the page gives no approximation); no biases (Eq. 1/2 have none); the logit scale is a parameter,
  1.0 by default (Eq. 2 has no 1/sqrt(d_h)); exp is evaluated after subtracting
  the row maximum, an exact identity in real arithmetic that keeps fp64 finite;
  the cache holds n rows K = X W^K, V = X W^V; the plain step does not append the
  current token, the full step (``decode_layer_append``) does, for every head (see
  there); for a batch, S is the union of the per-token top-k sets and is
  used by every token; index sets are returned in ascending order; the top-k
  decision is taken on scores rounded to fp32, the precision the kernel decides in.

Array conventions: inputs are NumPy arrays in the storage layouts of
``contextual_sparsity_mlp_amd.synth``.  Floating arrays may be float32 or float64;
a uint16 array is read as bfloat16 bit patterns and widened exactly (bits << 16);
weight-only fp8 matrices come as ``Fp8Rows`` (E4M3 codes and one scale per row),
widened exactly to scale * value.  The pages endorse weight-only quantization for
decode without fixing a format (the Deja Vu page, section 1, checks the method's
compatibility with quantization; the survey page's quantization section credits
weight-only quantization with faster decoding because fewer weight bytes leave
HBM); the reading here is the OCP E4M3 format with a per-row scale.
Rows are gathered before widening, so a full OPT-175B-shaped layer needs only its
selected rows in float64.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------- #
# Exact widening of stored values                                             #
# --------------------------------------------------------------------------- #


def decode_e4m3(codes) -> np.ndarray:
    """Value of fp8 E4M3 codes (the OCP 8-bit floating-point format: sign, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal, m/8 * 2^-6;
    S.1111.111 is NaN; no infinities), exactly, as float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * val
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, val)


class Fp8Rows:
    """Weight-only fp8 storage: codes [..., d] (uint8, E4M3) with one scale per row
    ([...], float); element = scale[row] * decode(code).  Indexing gathers rows."""

    def __init__(self, codes, scales):
        self.codes = np.asarray(codes, dtype=np.uint8)
        self.scales = np.asarray(scales)
        assert self.codes.shape[:-1] == self.scales.shape

    def __getitem__(self, idx):
        return Fp8Rows(self.codes[idx], self.scales[idx])

    @property
    def shape(self):
        return self.codes.shape


def widen(a) -> np.ndarray:
    """Exact value of a stored array as float64 (bf16 bit patterns: bits << 16; fp8
    rows: scale * decoded code)."""
    if isinstance(a, Fp8Rows):
        return decode_e4m3(a.codes) * widen(a.scales)[..., None]
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


def rows(W, idx) -> np.ndarray:
    """Gather rows ``idx`` (first axis) of a stored array, then widen them."""
    idx = np.asarray(idx, dtype=np.int64)
    if isinstance(W, Fp8Rows):
        return widen(W[idx])
    return widen(np.asarray(W)[idx])


def as_set(S) -> np.ndarray:
    """An index set as a sorted array of unique int64 indices."""
    return np.unique(np.asarray(S, dtype=np.int64))


# --------------------------------------------------------------------------- #
# A1: low-rank predictor scores                                               #
# --------------------------------------------------------------------------- #


def predict_scores(y, A, Bm) -> np.ndarray:
    """Scores s_b = (y_b A) B for every token b.

    ``A`` is stored [r][d] (row t is the t-th rank vector, i.e. column t of the
    d x r factor), ``Bm`` is stored [r][N].  Returns float64 [B][N].
    """
    y = widen(y)
    A_math = widen(A).T            # d x r
    B_math = widen(Bm)             # r x N
    z = y @ A_math                 # [B][r]
    return z @ B_math              # [B][N]


# --------------------------------------------------------------------------- #
# A2: deterministic top-k and batch union                                     #
# --------------------------------------------------------------------------- #


def topk_row(s, k: int) -> np.ndarray:
    """The k indices of largest score, equal scores ordered by lower index first;
    returned ascending.  k <= 0 gives the empty set, k >= N gives all indices.

    -0.0 and +0.0 compare equal (ordinary float comparison).  Inputs must be finite.
    """
    s = np.asarray(s, dtype=np.float64)
    if not np.all(np.isfinite(s)):
        raise ValueError("top-k scores must be finite")
    N = s.shape[0]
    k = max(0, min(int(k), N))
    # Python's sort is stable and compares the key tuples lexicographically:
    # first by descending score, then by ascending index.
    order = sorted(range(N), key=lambda j: (-s[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def select_sets(scores, k: int, union: bool):
    """Per-token top-k of ``scores`` [B][N].

    union=True: one ascending array, the union over tokens.
    union=False: a list with one ascending array per token.
    """
    scores = np.asarray(scores)
    per_row = [topk_row(scores[b], k) for b in range(scores.shape[0])]
    if not union:
        return per_row
    out = np.zeros(0, dtype=np.int64)
    for p in per_row:
        out = np.union1d(out, p)
    return out.astype(np.int64)


def predict_and_select(y, A, Bm, k: int, union: bool):
    """Predictor scores, rounded to fp32 (the precision of the decision), then top-k."""
    s = predict_scores(y, A, Bm).astype(np.float32).astype(np.float64)
    return select_sets(s, k, union)


# --------------------------------------------------------------------------- #
# A3: sparse MLP, Eq. (1)                                                     #
# --------------------------------------------------------------------------- #


def relu(x):
    return np.maximum(x, 0.0)


def gelu(x):
    """GeLU(x) = x Phi(x), Phi(x) = (1 + erf(x / sqrt(2))) / 2 (float64 erf)."""
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def activation(name: str):
    """sigma by name: "relu" or "gelu"."""
    if name == "relu":
        return relu
    if name == "gelu":
        return gelu
    raise ValueError(f"unknown activation {name!r}")


def sparse_mlp(y, W1t, W2t, S_M, act: str = "relu") -> np.ndarray:
    """MLP_{S_M}(y) = sigma(y W1_{S_M}) (W2_{S_M})^T, sigma = ReLU or GeLU.

    W1t/W2t are stored neuron-major [F][d]: row i is the column W1_i / W2_i.
    Returns float64 [B][d].  An empty set gives exactly zero.
    """
    y = widen(y)
    S = as_set(S_M)
    W1_S = rows(W1t, S).T          # d x |S|   (columns W1_i, i in S)
    W2_S = rows(W2t, S).T          # d x |S|
    h = activation(act)(y @ W1_S)  # [B][|S|]
    return h @ W2_S.T              # [B][d]


# --------------------------------------------------------------------------- #
# A4: head-sparse decode attention, Eq. (2)                                   #
# --------------------------------------------------------------------------- #


def head_output(y_b, WQ_i, K_bi, V_bi, scale: float = 1.0) -> np.ndarray:
    """H_i(y) for one token: D^{-1} exp(scale * y W^Q (X W^K)^T) X W^V.

    WQ_i is W_i^Q (d x dh); K_bi = X W_i^K and V_bi = X W_i^V (n x dh).
    The maximum logit is subtracted before exp; numerator and D_i scale alike.
    """
    q = y_b @ WQ_i                         # dh
    logits = scale * (q @ K_bi.T)          # n
    e = np.exp(logits - logits.max())
    D = e.sum()
    return (e @ V_bi) / D                  # dh


def sparse_mha(y, Wq, Wo, K, V, S_A, scale: float = 1.0) -> np.ndarray:
    """MHA_{S_A}(y) = sum_{i in S_A} H_i(y) W_i^O for each token of the batch.

    Wq, Wo stored [h][dh][d]: W_i^Q = Wq[i]^T (d x dh), W_i^O = Wo[i] (dh x d).
    K, V stored [B][h][n][dh]: token b attends over its own cache.
    Returns float64 [B][d].  An empty set gives exactly zero.
    """
    y = widen(y)
    B, d = y.shape
    out = np.zeros((B, d), dtype=np.float64)
    for i in as_set(S_A):
        WQ_i = rows(Wq, [i])[0].T
        WO_i = rows(Wo, [i])[0]
        for b in range(B):
            H = head_output(y[b], WQ_i, widen(np.asarray(K)[b, i]), widen(np.asarray(V)[b, i]),
                            scale)
            out[b] += H @ WO_i
    return out


# --------------------------------------------------------------------------- #
# A5: one decode layer with the layer-ahead predictor                         #
# --------------------------------------------------------------------------- #


def decode_layer(y, layer: dict, S_M, S_A, next_layer: dict | None, scale: float = 1.0):
    """y_{l+1} = y_l + MLP_{S_M}(y_l) + MHA_{S_A}(y_l); both blocks read y_l.

    The sets of layer l+1 are predicted from y_l (the layer's input, not its
    output) with layer l+1's predictor: the asynchronous look-ahead.
    ``layer`` / ``next_layer`` hold W1t, W2t, Wq, Wo, K, V and, for the
    predictor, A_M, B_M, A_A, B_A, k_m, k_a, union; "act" (default "relu") names
    the MLP's activation.
    Returns (y_next float64 [B][d], (S_M_next, S_A_next) or None).
    """
    yy = widen(y)
    mlp = sparse_mlp(yy, layer["W1t"], layer["W2t"], S_M, layer.get("act", "relu"))
    mha = sparse_mha(yy, layer["Wq"], layer["Wo"], layer["K"], layer["V"], S_A, scale)
    y_next = yy + mlp + mha
    sets = None
    if next_layer is not None:
        sets = (predict_and_select(yy, next_layer["A_M"], next_layer["B_M"],
                                   next_layer["k_m"], next_layer["union"]),
                predict_and_select(yy, next_layer["A_A"], next_layer["B_A"],
                                   next_layer["k_a"], next_layer["union"]))
    return y_next, sets


# --------------------------------------------------------------------------- #
# The full decode step: the current token's keys and values join the cache    #
# --------------------------------------------------------------------------- #


def round_bf16(x) -> np.ndarray:
    """float64 values rounded to the nearest bfloat16 (8 significant bits, ties to
    even, bf16 subnormals below 2^-126 on the 2^-133 grid), as bf16 bit patterns
    (uint16).  Rounds once, from the float64 value."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                        # |x| = m 2^e with 0.5 <= m < 1
    e = np.maximum(e, -125)                   # bf16 normals start at 2^-126 = 0.5 * 2^-125
    q = np.rint(np.ldexp(x, 8 - e))           # 8 significant bits; rint ties to even
    v = np.ldexp(q, e - 8).astype(np.float32)   # exact: v has at most 8 significant bits
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def store_as(x, like) -> np.ndarray:
    """float64 values rounded to the storage type of array ``like`` (bf16 bit
    patterns for uint16, else float32 or float64)."""
    dt = np.asarray(like).dtype
    if dt == np.uint16:
        return round_bf16(x)
    return np.asarray(x, dtype=np.float64).astype(dt)


def kv_for_token(y, Wk, Wv):
    """k_i = y W_i^K and v_i = y W_i^V of the current token for every head i
    (float64 [B][h][dh]); Wk, Wv are stored like Wq: [h][dh][d], row c of head i
    holding column c of W_i^K (W_i^V).  Eq. (2) builds K = X W^K, V = X W^V from
    the rows of X; these are the current token's rows."""
    y = widen(y)
    WK, WV = widen(Wk), widen(Wv)
    h, dh, d = WK.shape
    k = (WK.reshape(h * dh, d) @ y.T).T.reshape(-1, h, dh)
    v = (WV.reshape(h * dh, d) @ y.T).T.reshape(-1, h, dh)
    return k, v


def decode_layer_append(y, layer: dict, S_M, S_A, next_layer: dict | None, n: int,
                        scale: float = 1.0):
    """One decode step that also extends the KV cache (the KV-cache blog page,
    figure (b): at a decode step the current token's key and value join the
    stored ones, attention runs over all of them, and they are then kept).

    Readings (the pages say nothing of heads a step skips): X in Eq. (2) holds
    every previous token for every head, so the current token's k and v are
    computed and stored for all h heads, selected or not; they are stored at row
    n of each head's cache, rounded to the cache's storage type, and the selected
    heads attend over rows 0..n, the current token's own stored row among them.

    ``layer`` holds the decode layer's arrays plus Wk, Wv; K, V are [B][h][cap][dh]
    with cap > n, of which rows 0..n-1 are the cache (rows n and beyond are not
    read).  Returns (y_next, sets, (k_row, v_row)): the layer output and next sets
    as ``decode_layer`` gives them, and the stored rows [B][h][dh] in the cache's
    storage type.
    """
    K, V = np.asarray(layer["K"]), np.asarray(layer["V"])
    if not 0 <= n < K.shape[2]:
        raise ValueError(f"row {n} is outside a cache of {K.shape[2]} rows")
    k, v = kv_for_token(y, layer["Wk"], layer["Wv"])
    k_row, v_row = store_as(k, K), store_as(v, V)
    K1 = np.concatenate([K[:, :, :n], k_row[:, :, None, :]], axis=2)
    V1 = np.concatenate([V[:, :, :n], v_row[:, :, None, :]], axis=2)
    y_next, sets = decode_layer(y, dict(layer, K=K1, V=V1), S_M, S_A, next_layer, scale)
    return y_next, sets, (k_row, v_row)


def decode_stack(y0, layers: list, scale: float = 1.0):
    """Run a stack of decode layers with the look-ahead schedule.

    Layer 0's sets come from its own predictor applied to y_0 (nothing runs
    ahead of it); every later layer's sets come from the previous layer's input.
    Returns (y_L, list of (S_M, S_A) used by each layer).
    """
    y = widen(y0)
    L0 = layers[0]
    sets = (predict_and_select(y, L0["A_M"], L0["B_M"], L0["k_m"], L0["union"]),
            predict_and_select(y, L0["A_A"], L0["B_A"], L0["k_a"], L0["union"]))
    used = []
    for l, layer in enumerate(layers):
        nxt = layers[l + 1] if l + 1 < len(layers) else None
        used.append(sets)
        y, sets = decode_layer(y, layer, sets[0], sets[1], nxt, scale)
    return y, used
