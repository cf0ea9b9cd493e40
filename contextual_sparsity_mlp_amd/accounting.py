"""Algorithmic bytes and flops of the decode step (host arithmetic for reporting).

"Algorithmic" means what the method must move, not what a kernel happens to
fetch: each selected row, head weight and cached key/value is counted once, in
its stored width.  Counted per decode layer, with the actual (union) set sizes.

Sources for what is read: Deja Vu page, section 2.3, Eq. (1) reads W1_i and W2_i
for i in S_M; Eq. (2) reads W_i^Q, W_i^O for i in S_A and the cached X W_i^K,
X W_i^V of every token; the predictor reads both low-rank factors in full.
KV size per token follows the survey-notes page (KV cache sizing): 2 tensors x
hidden width x layers x bytes per element.
"""
from __future__ import annotations

from dataclasses import dataclass


def kv_bytes_per_token(hidden: int, layers: int, bytes_per_elem: int = 2) -> int:
    """K and V of one token across layers: 2 * hidden * layers * bytes."""
    return 2 * hidden * layers * bytes_per_elem


@dataclass
class StepBytes:
    mlp: int            # W1 and W2 rows of S_M
    attn_weights: int   # W^Q and W^O rows of S_A
    kv: int             # K and V rows of S_A for every token
    io: int             # y in, y out (and the MLP partial the combine reads)
    predictor: int      # A_M, B_M, A_A, B_A in full
    append: int = 0     # the KV append: W^K, W^V rows of every head, the rows written

    @property
    def selected(self) -> int:
        """Everything the layer step moves except the predictor."""
        return self.mlp + self.attn_weights + self.kv + self.io + self.append

    @property
    def total(self) -> int:
        return self.selected + self.predictor


def step_bytes(*, batch: int, d: int, F: int, h: int, dh: int, n_ctx: int, r: int, u_m: int,
               u_a: int, w_bytes: int = 2, kv_bytes: int = 2, with_predictor: bool = True,
               p_bytes: int | None = None, row_scale_bytes: int = 0,
               kv_append: bool = False) -> StepBytes:
    """Algorithmic bytes of one step.  w_bytes per selected weight element (1 for
    weight-only fp8, whose rows also carry row_scale_bytes of scale each); p_bytes per
    predictor element (default w_bytes).  kv_append: the step also computes every
    head's k and v of the current token (W^K and W^V read in full), writes them to
    row n_ctx of the cache and attends over n_ctx + 1 rows."""
    row = d * w_bytes + row_scale_bytes
    mlp = u_m * 2 * row
    attn_w = u_a * 2 * dh * row
    n_att = n_ctx + (1 if kv_append else 0)
    kv = batch * u_a * 2 * n_att * dh * kv_bytes
    io = 2 * batch * d * 4
    pb = w_bytes if p_bytes is None else p_bytes
    pred = (2 * d * r + r * F + r * h) * pb if with_predictor else 0
    app = (2 * h * dh * row + 2 * batch * h * dh * kv_bytes) if kv_append else 0
    return StepBytes(mlp, attn_w, kv, io, pred, app)


def step_flops(*, batch: int, d: int, F: int, h: int, dh: int, n_ctx: int, r: int, u_m: int,
               u_a: int, with_predictor: bool = True) -> int:
    f = batch * (4 * d * u_m + u_a * (4 * d * dh + 4 * n_ctx * dh))
    if with_predictor:
        f += batch * 2 * (2 * d * r + r * F + r * h)
    return f


def phase_bytes(*, batch: int, d: int, F: int, h: int, dh: int, n_ctx: int, r: int, u_m: int,
                u_a: int, w_bytes: int = 2, kv_bytes: int = 2, with_predictor: bool = True,
                p_bytes: int | None = None, row_scale_bytes: int = 0, sparse_launches: int = 2,
                kv_append: bool = False, lookahead_launches: int = 3):
    """Bytes each launch of the decode layer must move.

    With the predictor (the look-ahead step), three launches:
      1 gathered row dots: W1 rows, W^Q rows, predictor A factors, y;
      2 attention beside the predictor's second factors: K/V of the selected heads,
        predictor B factors;
      3 one row sum over W2 and W^O rows, combined with y_in into y_out, beside the
        next layer's top-k: W2 rows, W^O rows, y_in read, y_out written, scores read.
    or five (lookahead_launches=5: the predictor's row sums on the matrix cores, for a
    batch): the attention alone, the predictor B factors, then the score histograms
    (the scores read) before the row sum and top-k.
    Without it (the sparse MLP + MHA alone), one launch (sparse_launches=1) that
    streams everything: W1, W^Q, W2 and W^O rows, K/V, y_in read, y_out written; or
    two launches:
      1 gathered row dots: W1 rows, W^Q rows, y;
      2 attention, and the row sum over W2 then W^O rows: K/V, W2 rows, W^O rows,
        y_in read, y_out written.
    or, when the attention cannot share the row sum's launch (fp8 rows, larger
    batches: sparse_launches=3), row dots, attention alone (K/V), then the row sum.
    With kv_append the row dots also read W^K and W^V in full and write the cache
    rows, and the attention reads n_ctx + 1 rows.
    Small intermediates handed between launches (row dots, q, head outputs, attention
    pieces, scores written: under 1 MB at batch 1) are not counted.
    """
    row = d * w_bytes + row_scale_bytes
    pb = w_bytes if p_bytes is None else p_bytes
    p1 = u_m * row + u_a * dh * row + batch * d * 4
    n_att = n_ctx + (1 if kv_append else 0)
    kv = batch * u_a * 2 * n_att * dh * kv_bytes
    if kv_append:
        p1 += 2 * h * dh * row + 2 * batch * h * dh * kv_bytes
    out = u_m * row + u_a * dh * row + 2 * batch * d * 4
    if not with_predictor:
        if sparse_launches == 1:
            return [p1 - batch * d * 4 + kv + out]
        return [p1, kv, out] if sparse_launches == 3 else [p1, kv + out]
    p1 += 2 * r * d * pb
    p2 = kv + (r * F + r * h) * pb
    p3 = out + batch * (F + h) * 4
    if lookahead_launches == 5:
        return [p1, kv, (r * F + r * h) * pb, batch * (F + h) * 4, p3]
    return [p1, p2, p3]
