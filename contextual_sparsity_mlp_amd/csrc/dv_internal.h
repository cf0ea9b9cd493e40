// dv_internal.h - task descriptors shared by the host planner (dv_api.hip) and the
// device code (dv_kernels.hip).  Not part of the public ABI.
//
// The decode step is expressed with four device routines that each cover one
// access pattern of the Deja Vu step (page "Deja Vu: contextual sparsity for
// efficient LLMs at inference time", section 2.3, Eq. (1) and (2)):
//   rowdot : out[b][s] = y[b] . R[row(s)]        gathered rows dotted with the input
//            (W1_i of Eq. 1, columns of W_i^Q of Eq. 2, predictor factor A)
//   axpy   : out[b]   = sum_s c[b][s] * R[row(s)] gathered rows scaled and summed
//            (W2_i of Eq. 1 with c = ReLU(a), rows of W_i^O of Eq. 2, factor Bm)
//   attn   : softmax(scale q K^T) V per selected head, the n-loop of Eq. (2)
//   select : per-row top-k by radix select, and the union of rows
// A launch ("phase") runs any mix of them; each block picks its routine from its
// index, so independent work shares one grid and one launch.
#pragma once

#include <stdint.h>

namespace dv {

constexpr int kThreads = 256;            // threads per block, every kernel
constexpr int kWaves = kThreads / 64;    // wave64
constexpr int kMaxSeg = 4;               // segments per rowdot / axpy task
constexpr int kMaxChunks = 64;           // row chunks per axpy segment (partials bound)
constexpr int kMaxSplit = 64;            // key splits per (token, head)
constexpr int kAttnMaxKeys = 2048;       // keys per attention block (logits in LDS)
constexpr int kLdsBudget = 64 * 1024;    // dynamic LDS per block
constexpr int kSelectTile = kThreads * 16;   // elements per selection tile
constexpr int kUnionWordsPerThread = 4;

enum : int { W_F32 = 0, W_BF16 = 1 };

// A logical list of rows: slot s < count expands to rows idx[s]*expand + e, e < expand.
struct RowList {
  const int32_t* idx;      // nullptr: slot s is item s
  const int32_t* count;    // device count of slots; nullptr: host_count slots
  int host_count;          // capacity (slots); the device count is clamped to it
  int expand;              // rows per slot (dh for heads, 1 otherwise)
  int items;               // valid item indices are [0, items)
};

struct RowdotSeg {
  const void* W;           // row (item*expand + e) starts at W + that * row_stride elements
  long long row_stride;    // elements
  int wdt;
  RowList rows;
  float* out;              // out[b * out_ld + s*expand + e]
  int out_ld;
  int cap;                 // capacity in logical rows = host_count * expand
};

struct RowdotTask {
  RowdotSeg seg[kMaxSeg];
  int nseg;
  const float* y;          // [batch][d]
  int batch, d;
  int bt_lds;              // tokens of y staged in LDS at once (<= BT template)
  int blocks;
  uint32_t* zero_ptr;      // counters used by later launches of the same call
  int zero_words;
};

struct AxpySeg {
  const void* W;
  long long row_stride;    // elements
  int wdt;
  RowList rows;
  const float* coef;       // coef[b * coef_ld + s*expand + e]
  int coef_ld;
  int relu;                // use max(coef, 0)
  int ncols;               // output columns
  int vec;                 // elements per thread per row (8 bf16 / 4 f32 / 1 scalar)
  int nslices, nchunks, nbt;
  int block0;              // first block of this segment inside the task
  float* partial;          // [nbt][nchunks][BT][ncols]
  uint32_t* tickets;       // [nbt][nslices], zero on entry
  float* out;              // out[b * out_ld + col]
  int out_ld;
  const float* add0;       // optional addends [b * add_ld + col]
  const float* add1;
  int add_ld;
  int accumulate;          // add the previous value of out
};

struct AxpyTask {
  AxpySeg seg[kMaxSeg];
  int nseg;
  int batch;
  int blocks;
};

struct AttnTask {
  const float* q;          // q[b * q_ld + s*dh + c]
  int q_ld;
  const void* K;           // [batch][h][n][dh]
  const void* V;
  int kvdt;
  int batch, h, n, dh;
  RowList heads;           // expand = 1, items = h
  float scale;
  int nsplit, per;         // key splits per (token, slot), keys per split
  float* part;             // [batch][cap][nsplit][dh + 2]: m, l, o[dh]
  uint32_t* tickets;       // [batch][cap], zero on entry
  float* o;                // o[b * o_ld + s*dh + c]
  int o_ld;
  int blocks;              // batch * cap * nsplit
};

struct SelectProblem {
  const float* scores;     // row b at scores + b * ld
  int ld, N, k;
  int mode;                // 0: ascending indices at idx + b*k, count[b]; 1: bitmask rows
  int32_t* idx;
  int32_t* count;
  uint32_t* bits;          // [batch][nwords]
  int nwords;
};

struct SelectTask {
  SelectProblem p[2];
  int np, batch, blocks;   // blocks = np * batch
};

struct UnionProblem {
  const uint32_t* bits;    // [batch][nwords]
  int nwords, N, batch;
  int32_t* idx;
  int32_t* count;
};

struct UnionTask {
  UnionProblem p[2];
  int np, blocks;
};

enum : int { T_ROWDOT = 1, T_ATTN = 2, T_AXPY = 4, T_SELECT = 8, T_UNION = 16 };

struct PhaseArgs {
  RowdotTask rowdot;
  AttnTask attn;
  AxpyTask axpy;
  SelectTask select;
  UnionTask uni;
  int b_rowdot, b_attn, b_axpy, b_select, b_union;   // first block of each task
};

// Host-side launcher implemented in dv_kernels.hip.  Returns a hipError_t as int.
int launch_phase(int flags, int bt, const PhaseArgs& a, int grid, int lds_bytes, void* stream);

}  // namespace dv
