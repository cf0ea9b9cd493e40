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
//   top-k  : per-row exact top-k (histogram, classify, resolve) and the batch union
// A launch ("phase") runs any mix of them; each block picks its routine from its
// index, so independent work shares one grid and one launch.
#pragma once

#include <stdint.h>

namespace dv {

constexpr int kThreads = 256;            // threads per block, every kernel
constexpr int kWaves = kThreads / 64;    // wave64
constexpr int kMaxSeg = 4;               // segments per rowdot / axpy task
constexpr int kMaxRowdotSeg = 6;         // row-dot segments of a launch that also stores
                                         //   the current token's k and v (T_KV)
constexpr int kMaxChunks = 32;           // row chunks per axpy segment (partials bound)
constexpr int kAxSliceLanes = 32;        // lanes across the columns of one axpy slice
constexpr int kAxGroups = 8;             // row groups (half-waves) per axpy block
constexpr int kAxpyTileRows = 512;       // axpy rows whose ids / coefficients sit in LDS
constexpr int kAxPackedU = 6;            // axpy bf16 rows in flight per row group
constexpr int kAxPrefetchU = 6;          //   of which loaded before a wait (one-tile path)
constexpr int kAxFp8WaitU = 8;           //   fp8 rows in the waiting launch
constexpr double kWoChunkShare = 0.40;   // row-sum chunks given to W^O rows (waiting launch)
// In-launch counters sit one per 256-byte line (same-address atomics and polls
// serialise); the counter of index c is ctr[c * kCtrStride].
constexpr int kCtrStride = 64;
constexpr int kMaxSplit = 64;            // key splits per (token, head)
constexpr int kLdsBudget = 64 * 1024;    // dynamic LDS per block
constexpr int kTopShift = 20;            // first-level digit: the top 12 bits of a score key
constexpr int kHistBins = 1 << (32 - kTopShift);
constexpr int kLowBins = 1024;           // the remaining 20 bits: two 10-bit digits
constexpr int kSegElems = kThreads * 8;  // scores per top-k classify block
constexpr int kCandPerThread = 8;        // candidates a resolving thread holds in registers
constexpr int kCandTile = kThreads * kCandPerThread;
constexpr int kResolveWords = 1536;      // bitmask words a resolving block keeps in LDS (N <= 49152)
constexpr int kMaxSegs = 256;            // classify segments per row (N <= 524288)
constexpr int kWordsPerThread = 4;       // bitmask words per thread when compacting
constexpr int kMfmaRows = 16;            // matrix-core row dots: rows per tile and tokens per token tile
constexpr int kMfmaRT = 2;               //   row tiles per block unit
constexpr int kMfmaCols = 128;           //   columns per step (4 MFMA k-steps of 32); d % 128 == 0
constexpr int kMfmaMinBatch = 2;         //   smallest batch that takes them (row dots)
constexpr int kAxmTile = 256;           //   row sums: rows whose ids / coefficients sit in LDS (2 groups a wave)
constexpr int kAxMfmaMinBatch = 3;       //   row sums (measured: batch 4 row sum 187 -> 130 us)
constexpr int kMfmaBlocksPerCu = 3;      //   resident blocks per CU the grid is sized for (137 VGPRs)
constexpr int kMfmaLdsBlocksPerCu = 3;   //   the same for the row dots with y in LDS (32 tokens; 16: one more)

enum : int { W_F32 = 0, W_BF16 = 1, W_FP8 = 2 };   // W_FP8: E4M3 codes, one scale per row
enum : int { A_NONE = 0, A_RELU = 1, A_GELU = 2 };   // row-sum coefficient activations

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
  RowdotSeg seg[kMaxRowdotSeg];      // launches without T_KV use the first kMaxSeg
  const float* seg_scale[kMaxRowdotSeg];   // W_FP8 segments: scale of row (item*expand + e)
  // T_KV segments: instead of out, the dot of row (item*expand + e) with token b is
  // stored in the cache's type at seg_store + b*store_ld_b + item*store_ld_item + e
  void* seg_store[kMaxRowdotSeg];
  long long store_ld_b;
  long long store_ld_item;
  int store_dt;            // W_BF16 or W_F32
  int nseg;
  const float* y;          // [batch][d]
  int batch, d;
  int bt_lds;              // tokens of y staged in LDS at once (<= BT template)
  int mfma_nt;             // the matrix-core row dots (bf16 rows only, no cache stores):
                           //   1 / 2: mfma_nt token tiles of 16, y from L2; 3 / 4: batch
                           //   <= 16 / 32, y staged in LDS; 0: one wave per row
  int mfma_parts;          // mfma_nt 3, 4: column parts per 128-row unit (1: no partials)
  float* mfma_partial;     // [unit][part][2048 per 16 tokens] partial tiles
  uint32_t* mfma_tickets;  // [unit] parts finished, zero on entry
  int mfma_ticket_words;
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
  int act;                 // activation applied to each coefficient: A_NONE, A_RELU, A_GELU
  // Optional second row source summed into the same columns (same stride and
  // dtype): its rows follow the first source's rows in the row order.
  const void* W2;          // nullptr: one source
  RowList rows2;
  const float* coef2;
  int coef2_ld;
  int act2;
  int ncols;               // output columns
  int vec;                 // elements per thread per row (8 bf16 / 4 f32 / 1 scalar)
  int mfma_nt;             // 1 / 2: matrix-core blocks with 16 / 32 tokens per block tile
                           //   (bf16 rows, 128-column slices); 0: the wave path
  int nslices, nchunks, nbt;
  int block0;              // first block of this segment inside the task
  float* partial;          // [nbt][nchunks][BT][ncols]
  uint32_t* tickets;       // [nbt][nslices], zero on entry
  uint32_t* hist;          // optional [batch][kHistBins]: top-digit histogram of the output
  float* out;              // out[b * out_ld + col]
  int out_ld;
  const float* add0;       // optional addends [b * add_ld + col]
  const float* add1;
  int add_ld;
  int accumulate;          // add the previous value of out
  // Hand-off inside one launch (all blocks resident): before the second-source rows
  // of slot s a block waits until wait_ctr[s * kCtrStride] >= wait_target; coef2 is
  // then read coherently.  (The block's share of the second source is taken one slot
  // at a time, so it waits only on the slots its rows belong to.)
  const uint32_t* wait_ctr;
  uint32_t wait_target;
};

struct AxpyTask {
  uint32_t spins;          // bounded waits (AxpySeg::wait_ctr): poll limit
  uint32_t* fault;         // device word a wait that gave up marks (see dv_check)
  AxpySeg seg[kMaxSeg];
  // W_FP8 segments: per-row scales of the first / second source (row item*expand + e),
  // folded into the coefficients; kept apart from AxpySeg, whose by-value selection
  // costs scalar registers in every launch mix
  const float* seg_scale[kMaxSeg][2];
  // Waiting segments (wait_ctr) whose second-source coefficients are attention
  // outputs left as per-split softmax pieces (AttnTask::part_only): the pieces
  // [batch][rows2.host_count][nsplit2][rows2.expand + 2], combined by the row-sum
  // block as it stages the coefficients; nullptr: coef2 holds the coefficients.
  const float* part2;
  int nsplit2;
  // Waiting segments: c2 > 0 gives the last c2 row chunks of each column slice the
  // second source's rows alone (its rows split c2 ways) and the others the first
  // source's rows alone; 0: every chunk takes its share of both, first source first.
  int c2;
  // Row sums without waits: chunk c of C takes a share of the rows weighted
  // skew (C-1-c) + 8 (C-1) (0: equal shares), so the blocks dispatched first, which
  // stream faster on their CU, take more.
  int skew;
  int nseg;
  int batch;
  int blocks;
};

struct AttnTask {
  const float* q;          // q[b * q_ld + s*dh + c]
  int q_ld;
  const void* K;           // [batch][h][cap][dh]; rows 0..n-1 are attended
  const void* V;
  int kvdt;
  int batch, h, n, dh;
  int cap;                 // rows per (token, head) in K and V
  RowList heads;           // expand = 1, items = h
  float scale;
  int nsplit, per;         // key splits per (token, slot), keys per split
  float* part;             // [batch][cap][nsplit][dh + 2]: m, l, o[dh] of each split
                           //   (stored coherently)
  uint32_t* tickets;       // [batch][cap], zero on entry: the last split combines the
                           //   pieces into o
  float* o;                // o[b * o_ld + s*dh + c], stored coherently
  int o_ld;
  int blocks;              // batch * cap * nsplit
  int part_only;           // nsplit > 1: the splits only store their pieces (no combine;
                           //   every split reports its slot, see done_ctr)
  uint32_t* done_ctr;      // optional: done_ctr[s * kCtrStride] +1 for each token whose o
                           //   of slot s is stored, or with part_only for each stored
                           //   piece (after the stores)
};

// The sparse step in one launch (one token, bf16 rows, no next layer): every block is
// resident at once and works through one ordered queue of items,
//   dot items   4 gathered rows each (1 per wave) dotted with y: the W^Q rows of the
//               selected heads, then the W1 rows of the selected neurons;
//   attn items  one key split of one selected head;
//   sum items   one 256-column slice of a row sum: the W2 rows of one chunk of the
//               neuron list (coefficients sigma(a)), chunk-major, then the W^O rows of
//               one head (coefficients o), head-major.
// Queue order: W^Q dots, the first n_mfirst W1 dots (so that the first round of items,
// one per block, is all dots), the attention items (their heads' W^Q rows are dotted by
// the time blocks come back for a second item), the remaining W1 dots, the W2 sums,
// the W^O sums.  y sits in LDS for the dot items; the attention and sum scratch share
// that region, so a block stages y again before a dot item that follows an attention
// item (sum items come after every dot item).
// Item i belongs to queue i % kStreamQueues; the blocks of a queue take its items in
// order (each block starts with one of the first grid items and claims each later
// item of its queue from that queue's counter), so a block only waits for items taken
// before its own.  Readiness is counted per head (W^Q dots, attention) and per
// W1 chunk; each sum item stores its partial slice and the last one of a slice adds
// the partials in chunk order to y (fixed order: the result does not depend on which
// block took which item).
constexpr int kStreamRowsPerWave = 1;
constexpr int kStreamDotRows = kWaves * kStreamRowsPerWave;   // rows per dot item
constexpr int kStreamSlice = 256;                             // columns per sum item
constexpr int kStreamChunks = 16;                             // W2 chunks (target)
constexpr int kStreamU = 16;                                  // rows in flight per row group
constexpr int kStreamQueues = 8;                              // claim counters (item i: queue i % 8)

struct StreamTask {
  const void* W1; const void* W2; const void* Wq; const void* Wo;   // bf16 rows of d
  RowList LM;              // neurons: rows of W1t / W2t
  RowList LQ;              // heads, expand dh: rows of W^Q / W^O
  int d, dh, act;
  const float* y;          // [d] (a copy in the workspace when y_out is y)
  float* y_out;            // [d] = y + MLP + MHA
  float* a;                // [cap_m] W1 row dots
  float* q;                // [cap_a * dh] W^Q row dots (the attention's q)
  float* partial;          // [ncm + cap_a][d] partial slices of the row sum
  AttnTask at;             // attention of the selected heads, batch 1, tickets in the workspace
  uint32_t* ctr;           // counters (zeroed by the launch before), index c at c * kCtrStride:
                           //   [0, kStreamQueues) claims, then q_done[cap_a] (dot items per
                           //   head), m_done[ncm] (per W2 chunk), o_ready[cap_a], slice tickets
  int c_qdone, c_mdone, c_oready, c_stick;   // first counter index of each group
  int grid;                // a multiple of 64; block b serves queue (b / 8) % kStreamQueues
  int n_qi, n_mi, n_a;     // dot items over W^Q rows / W1 rows, attention items
  int n_mfirst;            // W1 dot items queued before the attention items
  int ncm, per_m;          // W2 chunks, rows per chunk (a multiple of kStreamDotRows)
  int nslice;              // column slices
  int n_items;
  int lds_union;           // bytes of the LDS region shared by y / sum / attention
  uint32_t spins, extra;   // bounded waits: poll limit; target offset (0 except in tests)
  uint32_t* fault;
};

// Exact top-k of score rows, in two steps that each spread over many blocks:
//   hist     12-bit top-digit histogram of every row (built by the blocks that
//            produce the scores, or by a launch of its own)
//   classify one block per (row, segment of kSegElems scores): finds the digit of
//            the k-th key from the histogram, marks keys above it in the row's
//            bitmask and lists the keys of that digit (index order) as candidates.
//            The last segment of a row to finish resolves the row: it picks the
//            needed candidates (lower index first on equal keys), ORs them into the
//            bitmask and compacts the ascending index list; with a batch union the
//            last row to be resolved ORs all rows.
struct TopkProblem {
  const float* scores;     // row b at scores + b * ld
  int ld, N, k, batch;
  int unite;               // 1: union of rows -> idx, count[0]; 0: row b -> idx + b*k, count[b]
  int32_t* idx;
  int32_t* count;
  uint32_t* hist;          // [batch][kHistBins], zero before it is built
  uint32_t* bits;          // [batch][nwords]
  int nwords;
  uint2* cand;             // [batch][nseg * kSegElems] (key, index) per segment
  int32_t* ccount;         // [batch][nseg] candidates per segment
  uint32_t* row_tickets;   // [batch] segments classified, zero before classify
  uint32_t* ticket;        // rows resolved (union), zero before classify
  int nseg;                // segments per row = ceil(N / kSegElems) <= kMaxSegs
};

struct TopkTask {
  TopkProblem p[2];
  int np;
  int blocks;
};

struct ZeroTask {
  uint32_t* ptr;
  int words;
  int blocks;
};

// T_WAIT: the row sums of the launch may wait for in-launch producers before their
// second source (see AxpySeg::wait_ctr) and combine attention pieces while staging.
// T_KV: the row dots of the launch include the current token's k and v, stored into
// the cache (RowdotTask::seg_store).
// T_FP8: the row dots and row sums of the launch may hold fp8 rows; the launches
// without it carry no fp8 code, which keeps their bf16 loops as tight as before.
// T_MFMA: some row sum of the launch runs on the matrix cores (AxpySeg::mfma_nt); set by
// the host launcher, so the wave-path launches keep their register budget.
// T_MFMA2: those row sums hold 32 tokens per block (mfma_nt 2).
enum : int { T_ROWDOT = 1, T_ATTN = 2, T_AXPY = 4, T_HIST = 8, T_CLASSIFY = 16, T_WAIT = 32,
             T_ZERO = 64, T_FP8 = 128, T_KV = 256, T_MFMA = 512, T_MFMA2 = 1024 };

struct PhaseArgs {
  RowdotTask rowdot;
  AttnTask attn;
  AxpyTask axpy;
  TopkTask topk;
  ZeroTask zero;
  int b_rowdot, b_attn, b_axpy, b_topk, b_zero;   // first block of each task
};

// Host-side launcher implemented in dv_kernels.hip.  Returns a hipError_t as int.
// ev0 / ev1 (hipEvent_t, may be null): events the runtime stamps with the kernel's own
// start and end (the launch's timing slot).
int launch_phase(int flags, int bt, const PhaseArgs& a, int grid, int lds_bytes, void* stream,
                 void* ev0 = nullptr, void* ev1 = nullptr);
// The one-launch sparse step (kvdt: W_BF16 or W_F32 cache); blocks per CU it keeps
// resident with lds_bytes of LDS (0 on error).
int launch_stream(int kvdt, const StreamTask& t, int grid, int lds_bytes, void* stream,
                  void* ev0 = nullptr, void* ev1 = nullptr);
int stream_occupancy(int kvdt, int lds_bytes);
// Device address of this device's fault word (set by in-launch waits that gave up);
// nullptr on error.  fault_take reads and clears it after synchronising `stream`.
uint32_t* fault_word();
int fault_take(void* stream, uint32_t* value);
// Blocks per CU of the kernel behind (flags, bt) that the runtime keeps resident with
// lds_bytes of dynamic LDS (0 for mixes it does not cover or on error).
int phase_occupancy(int flags, int bt, int lds_bytes);

}  // namespace dv
