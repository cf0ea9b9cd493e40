/*
 * dv.h - C ABI of the Deja Vu contextual-sparsity decode step for AMD MI355X (gfx950).
 *
 * The operations are those of "Deja Vu: contextual sparsity for efficient LLMs at
 * inference time" (Chinese translation page):
 *   - section 2.3, Eq. (1): sparse MLP  MLP_S(y) = sigma(y W1_S)(W2_S)^T, sigma = ReLU;
 *   - section 2.3, Eq. (2): head-sparse attention MHA_S(y) = sum_{i in S} H_i(y) W_i^O,
 *     H_i(y) = D_i(y)^{-1} exp(y W_i^Q (W_i^K)^T X^T) X W_i^V over a KV cache;
 *   - section 1 (contribution list): a low-overhead predictor that, from a layer's
 *     input, picks the next layer's neurons and heads, run one layer ahead (Fig. 2).
 *     Its form is not on the page; here it is low rank, s = (y A) B, followed by a
 *     deterministic top-k (lower index first on equal scores) and, for a batch, the
 *     union of the per-token sets.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates nothing; scratch space is the caller's workspace `ws` of `ws_bytes`
 *     bytes, sized with dv_workspace_bytes().  Workspace contents need no
 *     initialisation and are not meaningful between calls.
 *   - Layouts are row-major; a "row" is one contiguous d-vector:
 *       y, out      [batch][d]             fp32
 *       W1t, W2t    [F][d]                 row i = column i of W1 / W2 (neuron-major)
 *       Wq          [h][dh][d]             Wq[i][c] = column c of W_i^Q
 *       Wo          [h][dh][d]             Wo[i] = W_i^O (dh x d)
 *       K, V        [batch][h][n_ctx][dh]  K[b][i] = X_b W_i^K, V[b][i] = X_b W_i^V
 *       A           [r][d]                 predictor factor 1, one rank vector a row
 *       Bm          [r][N]                 predictor factor 2
 *       scores      [batch][N]             fp32
 *     Weights and KV are bf16 (DV_BF16) or fp32 (DV_F32); arithmetic is fp32.
 *   - Index lists are int32, ascending, with their length `count` in DEVICE memory.
 *     `max_count` is a host-side capacity used only to size grids; the device count
 *     is clamped to it.  Indices outside [0, F) or [0, h) contribute nothing.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream)
 *     and return once the work is enqueued.  They never synchronise with the device.
 *   - All argument checks run on the host before anything is enqueued: null pointers,
 *     sizes, d % 8 == 0, 16-byte alignment of every tensor pointer, k in [0, N],
 *     workspace size.  On failure nothing is enqueued and a negative code is returned;
 *     dv_last_error() then describes it.  A HIP error at enqueue (including one left
 *     by an earlier fault) returns DV_EHIP.
 *   - Results are deterministic: no floating-point atomics; reductions run in a fixed
 *     order, so equal inputs give bit-identical outputs.
 *   - Calls that share a workspace must not run concurrently.
 */
#ifndef DV_H
#define DV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  DV_FP8: weight-only fp8, the OCP E4M3 format (1 byte; sign, 4 exponent
 * bits with bias 7, 3 mantissa bits), with one fp32 scale per row: element =
 * scale[row] * value(code).  The pages endorse weight-only quantization for decode
 * (Deja Vu page, section 1; the survey page's quantization section) without naming a
 * format.  Only dv_decode_layer takes fp8 weights (W1t, W2t, Wq, Wo). */
typedef enum { DV_F32 = 0, DV_BF16 = 1, DV_FP8 = 2 } dv_dtype;

/* sigma of Eq. (1): the page names ReLU or GeLU (section 2.3, under Eq. (1)).  GeLU is
 * the exact x Phi(x) = x (1 + erf(x / sqrt 2)) / 2 (the page gives no approximation). */
typedef enum { DV_ACT_RELU = 0, DV_ACT_GELU = 1 } dv_act;

enum {
  DV_OK = 0,
  DV_EINVAL = -1,        /* bad argument: null pointer, size out of range, k not in [0, N] */
  DV_EALIGN = -2,        /* tensor pointer not 16-byte aligned, or d not a multiple of 8 */
  DV_EUNSUPPORTED = -3,  /* valid but unsupported shape (e.g. dh not in {32,64,128,256}) */
  DV_EWORKSPACE = -4,    /* ws NULL or ws_bytes smaller than dv_workspace_bytes() */
  DV_EHIP = -5,          /* the HIP runtime reported an error while enqueuing */
  DV_ETIMEOUT = -6       /* dv_check: a wait inside an earlier launch gave up */
};

/* Text describing the last non-OK return on the calling thread ("" if none). */
const char* dv_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int dv_version(void);

/* Operation codes for dv_workspace_bytes(). */
enum {
  DV_OP_PREDICT = 1,
  DV_OP_SELECT_TOPK = 2,
  DV_OP_SPARSE_MLP = 3,
  DV_OP_SPARSE_MHA = 4,
  DV_OP_DECODE_LAYER = 5
};

/* Shapes for workspace sizing.  Each operation reads the fields it uses:
 *   PREDICT:      batch, d, r, N
 *   SELECT_TOPK:  batch, N
 *   SPARSE_MLP:   batch, d, max_count_m
 *   SPARSE_MHA:   batch, d, dh, n_ctx, max_count_a
 *   DECODE_LAYER: batch, d, F, h, dh, n_ctx, r, max_count_m, max_count_a
 *                 (F, h, r describe the next layer's predictor as well) */
typedef struct {
  int batch;        /* tokens decoded together */
  int d;            /* model width */
  int F;            /* MLP neurons (4d in OPT) */
  int h;            /* attention heads */
  int dh;           /* head width */
  int n_ctx;        /* cached tokens per sequence (DECODE_LAYER: may be 0, for a step
                     * with the KV append on an empty cache) */
  int r;            /* predictor rank */
  int N;            /* items scored (PREDICT, SELECT_TOPK) */
  int max_count_m;  /* capacity of the neuron index list */
  int max_count_a;  /* capacity of the head index list */
} dv_shape;

/* Bytes of workspace the operation needs for these shapes (0 on invalid shapes,
 * with dv_last_error() set).  Pure host arithmetic: needs no GPU. */
size_t dv_workspace_bytes(int op, const dv_shape* shape);

/* A1 - low-rank predictor scores (Deja Vu page, section 1: a learned predictor
 * scores the next layer's neurons or heads from the layer input).
 *   scores[b][j] = sum_t ( sum_i y[b][i] A[t][i] ) Bm[t][j],   t < r, i < d, j < N.
 * y [batch][d] fp32; A [r][d] and Bm [r][N] in `wdt`; scores [batch][N] fp32 output. */
int dv_predict(const float* y, int batch, int d,
               const void* A, const void* Bm, int r, int N, dv_dtype wdt,
               float* scores, void* ws, size_t ws_bytes, void* stream);

/* A2 - deterministic top-k and batch union (Deja Vu page, section 2.3: choose the
 * sets under a compute budget).  For each row b, the k indices of largest score;
 * equal scores are taken lower index first; -0.0 equals +0.0.  Scores must be
 * finite (NaN ordering is unspecified).  k must be in [0, N].
 *   union_rows != 0: idx receives the ascending union over rows, capacity
 *                    min(N, batch * k); count[0] its length.
 *   union_rows == 0: row b's ascending set at idx + b * k; count[b] = k. */
int dv_select_topk(const float* scores, int batch, int N, int k, int union_rows,
                   int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/* A3 - sparse MLP, Deja Vu page section 2.3 Eq. (1), no bias:
 *   out[b] (+)= sum_{s < count} sigma(y[b] . W1t[idx[s]]) * W2t[idx[s]],
 * sigma = ReLU (act = DV_ACT_RELU) or GeLU (DV_ACT_GELU; any other value is
 * DV_EINVAL).  The set is shared by every token of the batch.  accumulate != 0 adds
 * to `out`, otherwise `out` is overwritten.  `out` must not alias `y`. */
int dv_sparse_mlp(const float* y, int batch, int d,
                  const void* W1t, const void* W2t, int F, dv_dtype wdt,
                  const int32_t* idx, const int32_t* count, int max_count,
                  float* out, int accumulate, int act, void* ws, size_t ws_bytes, void* stream);

/* A4 - head-sparse decode attention, Deja Vu page section 2.3 Eq. (2):
 *   q = y[b] W_i^Q,  t_j = scale * q . K[b][i][j],  p = softmax(t) over j < n_ctx,
 *   out[b] (+)= sum_{i in heads} (sum_j p_j V[b][i][j]) W_i^O.
 * Eq. (2) has no logit scale: pass 1.0 for it (a 1/sqrt(dh) may be passed or folded
 * into Wq).  The cache holds exactly n_ctx >= 1 tokens; nothing is appended.
 * dh must be one of 32, 64, 128, 256.  `out` must not alias `y`. */
int dv_sparse_mha(const float* y, int batch, int d, int h, int dh,
                  const void* Wq, const void* Wo, dv_dtype wdt,
                  const void* K, const void* V, int n_ctx, dv_dtype kvdt,
                  const int32_t* heads, const int32_t* count, int max_count, float scale,
                  float* out, int accumulate, void* ws, size_t ws_bytes, void* stream);

/* One decoder layer's tensors (device pointers) and predictor settings. */
typedef struct {
  int d, F, h, dh, n_ctx, r;
  int k_m, k_a;            /* per-token keep counts of this layer's predictor */
  dv_dtype wdt, kvdt;
  float scale;             /* attention logit scale (1.0 = Eq. (2) as written) */
  const void *W1t, *W2t, *Wq, *Wo;
  void *K, *V;             /* [batch][h][kv_cap][dh]; rows 0..n_ctx-1 are the cache (written
                            * only by the KV append, at row n_ctx) */
  const void *A_M, *B_M;   /* neuron predictor: [r][d], [r][F] */
  const void *A_A, *B_A;   /* head predictor:   [r][d], [r][h] */
  int act;                 /* sigma of this layer's MLP: dv_act (DV_ACT_RELU = 0) */
  dv_dtype pwdt;           /* A_M, B_M, A_A, B_A: DV_BF16 or DV_F32 (read from `next`) */
  /* wdt == DV_FP8: one fp32 scale per row of W1t [F], W2t [F], Wq [h*dh], Wo [h*dh]
   * (16-byte aligned; NULL otherwise) */
  const float *W1s, *W2s, *Wqs, *Wos;
  /* The full decode step with the KV append (KV-cache blog page, figure (b): the
   * current token's key and value join the cache and are attended with it).  When Wk
   * and Wv are both non-NULL, k_i = y W_i^K and v_i = y W_i^V of EVERY head i (a
   * reading: the pages say nothing of skipped heads, and Eq. (2)'s X holds every
   * token for every head) are stored, rounded to kvdt (bf16: nearest, ties to even),
   * at row n_ctx of each (token, head) cache; the heads of S_A then attend over rows
   * 0..n_ctx, the stored current row among them.  Wk, Wv: [h][dh][d] in wdt like Wq
   * (fp8: scales Wks, Wvs [h*dh], 16-byte aligned).  Both NULL: no append, rows
   * 0..n_ctx-1 attended (n_ctx may then not be 0).  The caller advances n_ctx between
   * steps.  Calls that append to the same cache rows must not overlap. */
  const void *Wk, *Wv;
  const float *Wks, *Wvs;
  int kv_cap;              /* rows per (token, head) of K and V; 0 means n_ctx.  With the
                            * append kv_cap > n_ctx (DV_EINVAL otherwise) */
} dv_layer;

/* A5 - one decode layer with the look-ahead predictor (Deja Vu page, section 1 and
 * Fig. 2: the predictor for layer l+1 runs on layer l's input):
 *   y_out = y_in + MLP_{S_M}(y_in) + MHA_{S_A}(y_in)       (both blocks read y_in)
 * and, when `next` is not NULL, next layer's sets from y_in:
 *   S_M' = union_b topk(predict(y_in; next->A_M, next->B_M), next->k_m), likewise S_A'.
 * (idx_m, count_m), (idx_a, count_a): this layer's sets (device), capacities max_count_m,
 * max_count_a.  next_idx_m needs capacity min(next->F, batch * next->k_m), next_idx_a
 * min(next->h, batch * next->k_a).  `next` must have the same d as `L`; its predictor
 * factors have type next->pwdt.  With L->wdt == DV_FP8 the layer's W1t, W2t, Wq, Wo are
 * fp8 rows with scales L->W1s, W2s, Wqs, Wos and d must be a multiple of 16
 * (DV_EALIGN otherwise); the KV cache stays L->kvdt.
 * y_out may equal y_in. */
int dv_decode_layer(const dv_layer* L, const dv_layer* next, int batch,
                    const float* y_in, float* y_out,
                    const int32_t* idx_m, const int32_t* count_m, int max_count_m,
                    const int32_t* idx_a, const int32_t* count_a, int max_count_a,
                    int32_t* next_idx_m, int32_t* next_count_m,
                    int32_t* next_idx_a, int32_t* next_count_a,
                    void* ws, size_t ws_bytes, void* stream);

/* dv_decode_layer without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, semantics and results as dv_decode_layer; the
 * workspace is instead a scratch array of dv_noalloc_scratch_bytes() bytes (64 MiB)
 * that the library holds on each device it runs on until the process ends.  Nothing
 * is allocated by the call.  Shapes whose workspace (dv_workspace_bytes with
 * DV_OP_DECODE_LAYER) exceeds the scratch are rejected with DV_EWORKSPACE before
 * anything is enqueued (a bf16 OPT-175B-shaped layer fits up to batch 2 with the
 * look-ahead predictor, up to batch 4 without it).  Every call on
 * one device shares that device's scratch: calls that may overlap on one device
 * (other streams, other threads) race and must be serialised by the caller. */
int dv_decode_layer_noalloc(const dv_layer* L, const dv_layer* next, int batch,
                            const float* y_in, float* y_out,
                            const int32_t* idx_m, const int32_t* count_m, int max_count_m,
                            const int32_t* idx_a, const int32_t* count_a, int max_count_a,
                            int32_t* next_idx_m, int32_t* next_count_m,
                            int32_t* next_idx_a, int32_t* next_count_a, void* stream);

/* Bytes of the scratch array behind dv_decode_layer_noalloc (per device). */
size_t dv_noalloc_scratch_bytes(void);

/* Reports what an asynchronous call cannot return: synchronises `stream`, then
 * returns DV_ETIMEOUT if a bounded wait inside a launch of an earlier call on this
 * device gave up (clearing that record), DV_EHIP if the HIP runtime reports an error,
 * else DV_OK.  Some launches hand values between their own blocks and wait for them
 * (they are sized so that all their blocks are resident at once); if that ever fails
 * to hold (another process on the device's compute units, a partitioned device), the
 * wait ends after a bounded number of polls and every output that depended on the
 * missing values is written as NaN, never as a silently wrong number. */
int dv_check(void* stream);

/* Test hook for that failure path: every later launch polls at most `spins` times per
 * wait (0 restores the default) and adds `extra` to each wait's target, so that with
 * extra > 0 every such wait gives up and its kernel still ends normally. */
int dv_debug_wait_limits(unsigned spins, unsigned extra);

/* Launch plan of dv_decode_layer / dv_decode_layer_noalloc for one token, bf16 rows, no
 * next-layer predictor and no cache append (the sparse MLP + head-sparse MHA step of
 * the Deja Vu page, section 2.3, Eq. (1) and (2), alone).  DV_PATH_TWO_LAUNCH: one
 * launch dots every gathered row, a second one runs attention and both row sums.
 * DV_PATH_ONE_LAUNCH: one launch whose resident blocks take the row dots, attention
 * items and row-sum slices from an ordered queue, each item waiting (bounded) on the
 * items it reads.  DV_PATH_AUTO (the default) takes the plan measured faster on
 * MI355X.  Both give the same results up to the rounding order of the row sums.
 * Other calls ignore the setting.  Returns DV_EINVAL for an unknown value. */
enum { DV_PATH_AUTO = 0, DV_PATH_TWO_LAUNCH = 1, DV_PATH_ONE_LAUNCH = 2 };
int dv_set_step_path(int path);

/* Phase timing for measurement.  dv_timing_enable(1) makes every later call record
 * a hipEvent pair for each of its kernel launches, which the runtime stamps with the
 * kernel's own start and end (hipExtLaunchKernelGGL; events are created here, once);
 * dv_timing_enable(0) stops recording.  dv_timing_read()
 * synchronises the recorded events and returns, per launch slot (the k-th launch
 * inside an entry point), the summed elapsed milliseconds and the number of launches
 * recorded, then clears the record.  At most `max_slots` slots are returned;
 * *n_slots receives the number filled. */
int dv_timing_enable(int on);
int dv_timing_read(float* ms_sum, int* launches, int max_slots, int* n_slots);

#ifdef __cplusplus
}
#endif

#endif /* DV_H */
