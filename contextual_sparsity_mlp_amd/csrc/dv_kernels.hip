// dv_kernels.hip - device code of the Deja Vu sparse decode step for gfx950.
//
// Four routines, each written for CDNA's 64-wide waves and 256-thread blocks:
//
//  rowdot  One wave owns one gathered row of d elements at a time and streams it
//          in 1 KiB wave-loads (16 B per lane), dotting it with the token inputs
//          staged once per block in LDS; the 64 lane partials are combined with
//          cross-lane shuffles.  Covers W1_i of Eq. (1), the d_h columns of a
//          selected W_i^Q of Eq. (2) and the predictor's first factor.
//  axpy    A block owns a (column slice x row chunk) tile.  Each thread keeps the
//          running sum of 8 (bf16) or 4 (fp32) output columns in registers across
//          the chunk's rows, reading 16 B per row; the chunk's row indices and
//          coefficients are staged in LDS and broadcast.  Partial sums go to the
//          workspace and the last block to finish a column slice (device-scope
//          ticket) adds the chunks in fixed order, so results are deterministic.
//          Covers W2_i scaled by ReLU(a_i) in Eq. (1), W_i^O scaled by H_i(y) in
//          Eq. (2) and the predictor's second factor.
//  attn    Decode attention over the cache for one (token, selected head, key
//          split): logits in LDS, max-subtracted exp, p.V, then the last split to
//          finish rescales and merges the splits (splitting the key axis follows
//          the Flash-Decoding idea named on the survey-notes page).
//  select  Exact top-k of one score row by a 4-pass 8-bit radix select on
//          order-preserving keys, then an index-ordered block scan that keeps the
//          lowest indices among keys equal to the threshold.  `union` ORs per-row
//          bitmasks and compacts them to an ascending list.
//
// No floating-point atomics anywhere; only integer tickets and LDS histograms.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dv_internal.h"

namespace dv {

// --------------------------------------------------------------------------- //
// helpers                                                                      //
// --------------------------------------------------------------------------- //

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& x, float (&f)[8]) {
  f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x);
  f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
  f[4] = bf16_lo(x.z); f[5] = bf16_hi(x.z);
  f[6] = bf16_lo(x.w); f[7] = bf16_hi(x.w);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Block-wide reductions over 256 threads; `scratch` holds kWaves floats.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += scratch[w];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float t = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t = fmaxf(t, scratch[w]);
  return t;
}

// Inclusive prefix sum over the 256 threads of a block, in thread order.
// `scratch` holds kWaves words; *total receives the block total.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t n = __shfl_up(v, off);
    if (lane >= off) v += n;
  }
  __syncthreads();
  if (lane == 63) scratch[wave] = v;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = scratch[w];
    before += (w < wave) ? s : 0u;
    tot += s;
  }
  *total = tot;
  return v + before;
}

// Number of valid slots of a row list (device count clamped to the capacity).
__device__ __forceinline__ int list_slots(const RowList& L) {
  int n = L.host_count;
  if (L.count) n = min(n, *L.count);
  return max(n, 0);
}

// Device-scope "last block to arrive" test: every thread calls it after writing
// its partial results; returns true in all threads of the last arriving block.
__device__ __forceinline__ bool arrive_last(uint32_t* ticket, uint32_t expected, int* flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = atomicAdd(ticket, 1u);
    *flag = (t == expected - 1u) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *flag != 0;
  if (last) __threadfence();
  return last;
}

// --------------------------------------------------------------------------- //
// rowdot                                                                       //
// --------------------------------------------------------------------------- //

__device__ __forceinline__ RowdotSeg rd_seg(const RowdotTask& T, int s) {
  switch (s) {
    case 0: return T.seg[0];
    case 1: return T.seg[1];
    case 2: return T.seg[2];
    default: return T.seg[3];
  }
}

// acc[b] += row . y_b for the lane's share of one bf16 row of d elements.
template <int BT, int U>
__device__ __forceinline__ void rowdot_bf16(const uint4* __restrict__ rp, const float* ylds, int d,
                                            int nb, int lane, float (&acc)[BT]) {
  const int nv = d >> 3;  // 16-byte vectors in the row
  for (int v0 = 0; v0 < nv; v0 += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 64 + lane;
      w[u] = (v < nv) ? rp[v] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 64 + lane;
      if (v < nv) {
        float f[8];
        unpack8(w[u], f);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b < nb) {
            const float4* yp = reinterpret_cast<const float4*>(ylds + b * d + v * 8);
            const float4 y0 = yp[0], y1 = yp[1];
            float a = acc[b];
            a = fmaf(f[0], y0.x, a); a = fmaf(f[1], y0.y, a);
            a = fmaf(f[2], y0.z, a); a = fmaf(f[3], y0.w, a);
            a = fmaf(f[4], y1.x, a); a = fmaf(f[5], y1.y, a);
            a = fmaf(f[6], y1.z, a); a = fmaf(f[7], y1.w, a);
            acc[b] = a;
          }
        }
      }
    }
  }
}

template <int BT, int U>
__device__ __forceinline__ void rowdot_f32(const float4* __restrict__ rp, const float* ylds, int d,
                                           int nb, int lane, float (&acc)[BT]) {
  const int nv = d >> 2;
  for (int v0 = 0; v0 < nv; v0 += 64 * U) {
    float4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 64 + lane;
      w[u] = (v < nv) ? rp[v] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 64 + lane;
      if (v < nv) {
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b < nb) {
            const float4 y0 = *reinterpret_cast<const float4*>(ylds + b * d + v * 4);
            float a = acc[b];
            a = fmaf(w[u].x, y0.x, a); a = fmaf(w[u].y, y0.y, a);
            a = fmaf(w[u].z, y0.z, a); a = fmaf(w[u].w, y0.w, a);
            acc[b] = a;
          }
        }
      }
    }
  }
}

template <int BT>
__device__ __forceinline__ void rowdot_task(const RowdotTask& T, int blk, float* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Counters used by later launches of the same call start at zero.
  for (int i = blk * kThreads + tid; i < T.zero_words; i += T.blocks * kThreads) T.zero_ptr[i] = 0u;

  int total_cap = 0;
#pragma unroll
  for (int s = 0; s < kMaxSeg; ++s) total_cap += (s < T.nseg) ? T.seg[s].cap : 0;
  const int total_waves = T.blocks * kWaves;
  const int gw = blk * kWaves + wave;
  const int d = T.d;

  for (int b0 = 0; b0 < T.batch; b0 += T.bt_lds) {
    const int nb = min(T.bt_lds, T.batch - b0);
    __syncthreads();
    {
      const float4* src = reinterpret_cast<const float4*>(T.y + (size_t)b0 * d);
      float4* dst = reinterpret_cast<float4*>(lds);
      const int n4 = (nb * d) >> 2;
      for (int i = tid; i < n4; i += kThreads) dst[i] = src[i];
    }
    __syncthreads();
    for (int g = gw; g < total_cap; g += total_waves) {
      int s = 0, r = g;
#pragma unroll
      for (int i = 0; i < kMaxSeg - 1; ++i) {
        const int c = T.seg[i].cap;
        if (s == i && r >= c) { r -= c; s = i + 1; }
      }
      const RowdotSeg S = rd_seg(T, s);
      const int ex = S.rows.expand;
      const int slot = (ex == 1) ? r : r / ex;
      const int e = (ex == 1) ? 0 : r - slot * ex;
      if (slot >= list_slots(S.rows)) continue;  // wave-uniform
      const int item = S.rows.idx ? S.rows.idx[slot] : slot;
      float acc[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[b] = 0.f;
      if ((unsigned)item < (unsigned)S.rows.items) {
        const long long row = (long long)item * ex + e;
        if (S.wdt == W_BF16) {
          const uint4* rp = reinterpret_cast<const uint4*>(
              static_cast<const uint16_t*>(S.W) + row * S.row_stride);
          rowdot_bf16<BT, 8>(rp, lds, d, nb, lane, acc);
        } else {
          const float4* rp = reinterpret_cast<const float4*>(
              static_cast<const float*>(S.W) + row * S.row_stride);
          rowdot_f32<BT, 8>(rp, lds, d, nb, lane, acc);
        }
      }
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[b] = wave_sum(acc[b]);
      if (lane == 0) {
#pragma unroll
        for (int b = 0; b < BT; ++b)
          if (b < nb) S.out[(size_t)(b0 + b) * S.out_ld + r] = acc[b];
      }
    }
  }
}

// --------------------------------------------------------------------------- //
// axpy                                                                         //
// --------------------------------------------------------------------------- //

constexpr int kAxpyTile = 256;   // rows whose indices / coefficients are staged at once

__device__ __forceinline__ AxpySeg ax_seg(const AxpyTask& T, int s) {
  switch (s) {
    case 0: return T.seg[0];
    case 1: return T.seg[1];
    case 2: return T.seg[2];
    default: return T.seg[3];
  }
}

template <int VEC, int WT>
__device__ __forceinline__ void load_cols(const void* W, long long off, float (&w)[VEC]) {
  if constexpr (WT == W_BF16 && VEC == 8) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + off), f);
#pragma unroll
    for (int v = 0; v < 8; ++v) w[v] = f[v];
  } else if constexpr (WT == W_F32 && VEC == 4) {
    const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + off);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (WT == W_BF16) {
    w[0] = __uint_as_float((uint32_t)(static_cast<const uint16_t*>(W)[off]) << 16);
  } else {
    w[0] = static_cast<const float*>(W)[off];
  }
}

// Accumulate rows [r0, r1) of the segment's list into acc (this thread's VEC columns).
template <int BT, int VEC, int WT>
__device__ __forceinline__ void axpy_rows(const AxpySeg& S, int r0, int r1, int b0, int nb,
                                          int col0, bool active, float* lds,
                                          float (&acc)[BT][VEC]) {
  constexpr int U = 8;
  int* lrow = reinterpret_cast<int*>(lds);                 // [kAxpyTile] row or -1
  float* lcoef = lds + kAxpyTile;                          // [BT][kAxpyTile]
  const int tid = threadIdx.x;
  const int ex = S.rows.expand;
  for (int t0 = r0; t0 < r1; t0 += kAxpyTile) {
    const int tn = min(kAxpyTile, r1 - t0);
    __syncthreads();
    for (int i = tid; i < tn; i += kThreads) {
      const int rr = t0 + i;
      const int slot = (ex == 1) ? rr : rr / ex;
      const int e = (ex == 1) ? 0 : rr - slot * ex;
      const int item = S.rows.idx ? S.rows.idx[slot] : slot;
      const bool ok = (unsigned)item < (unsigned)S.rows.items;
      lrow[i] = ok ? item * ex + e : -1;
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        float c = 0.f;
        if (ok && b < nb) {
          c = S.coef[(size_t)(b0 + b) * S.coef_ld + rr];
          if (S.relu) c = fmaxf(c, 0.f);
        }
        lcoef[b * kAxpyTile + i] = c;
      }
    }
    __syncthreads();
    if (active) {
      for (int i0 = 0; i0 < tn; i0 += U) {
        float w[U][VEC];
        float c[U][BT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u;
          const int row = (i < tn) ? lrow[i] : -1;
          if (row >= 0) {
            load_cols<VEC, WT>(S.W, (long long)row * S.row_stride + col0, w[u]);
          } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) w[u][v] = 0.f;
          }
#pragma unroll
          for (int b = 0; b < BT; ++b) c[u][b] = (i < tn) ? lcoef[b * kAxpyTile + i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int b = 0; b < BT; ++b)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[b][v] = fmaf(c[u][b], w[u][v], acc[b][v]);
      }
    }
  }
}

template <int BT, int VEC, int WT>
__device__ __forceinline__ void axpy_block(const AxpySeg& S, int lb, int batch, float* lds) {
  const int tid = threadIdx.x;
  const int chunk = lb % S.nchunks;
  const int rest = lb / S.nchunks;
  const int slice = rest % S.nslices;
  const int bti = rest / S.nslices;
  const int b0 = bti * BT;
  const int nb = min(BT, batch - b0);
  const int col0 = slice * (kThreads * VEC) + tid * VEC;
  const bool active = col0 < S.ncols;

  const int nrows = list_slots(S.rows) * S.rows.expand;
  const int per = (nrows + S.nchunks - 1) / S.nchunks;
  const int r0 = min(chunk * per, nrows);
  const int r1 = min(r0 + per, nrows);

  float acc[BT][VEC];
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[b][v] = 0.f;
  axpy_rows<BT, VEC, WT>(S, r0, r1, b0, nb, col0, active, lds, acc);

  const size_t ncols = (size_t)S.ncols;
  float* P = S.partial + (size_t)(bti * S.nchunks + chunk) * BT * ncols;
  if (active) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      if (b < nb) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) P[b * ncols + col0 + v] = acc[b][v];
      }
    }
  }
  int* flag = reinterpret_cast<int*>(lds);
  if (!arrive_last(&S.tickets[bti * S.nslices + slice], (uint32_t)S.nchunks, flag)) return;
  if (!active) return;
  const float* P0 = S.partial + (size_t)bti * S.nchunks * BT * ncols;
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    if (b < nb) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const size_t col = (size_t)col0 + v;
        float sum = 0.f;
        for (int c = 0; c < S.nchunks; ++c) sum += P0[((size_t)c * BT + b) * ncols + col];
        const size_t bo = (size_t)(b0 + b);
        if (S.add1) sum = S.add1[bo * S.add_ld + col] + sum;
        if (S.add0) sum = S.add0[bo * S.add_ld + col] + sum;
        float* o = S.out + bo * S.out_ld + col;
        if (S.accumulate) sum = *o + sum;
        *o = sum;
      }
    }
  }
}

template <int BT>
__device__ __forceinline__ void axpy_task(const AxpyTask& T, int blk, float* lds) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i)
    if (i < T.nseg && blk >= T.seg[i].block0) s = i;
  const AxpySeg S = ax_seg(T, s);
  const int lb = blk - S.block0;
  if (S.wdt == W_BF16) {
    if (S.vec == 8) axpy_block<BT, 8, W_BF16>(S, lb, T.batch, lds);
    else axpy_block<BT, 1, W_BF16>(S, lb, T.batch, lds);
  } else {
    if (S.vec == 4) axpy_block<BT, 4, W_F32>(S, lb, T.batch, lds);
    else axpy_block<BT, 1, W_F32>(S, lb, T.batch, lds);
  }
}

// --------------------------------------------------------------------------- //
// attention                                                                    //
// --------------------------------------------------------------------------- //

template <int WT>
__device__ __forceinline__ void attn_task(const AttnTask& T, int blk, float* lds) {
  constexpr int VEC = (WT == W_BF16) ? 8 : 4;
  constexpr int U = 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cap = T.heads.host_count;
  const int split = blk % T.nsplit;
  const int rest = blk / T.nsplit;
  const int slot = rest % cap;
  const int b = rest / cap;
  if (slot >= list_slots(T.heads)) return;
  const int head = T.heads.idx ? T.heads.idx[slot] : slot;
  if ((unsigned)head >= (unsigned)T.h) return;   // contributes nothing; W^O skips it too

  const int dh = T.dh;
  const int LPK = dh / VEC;          // lanes per key row
  const int KPW = 64 / LPK;          // keys per wave-load
  const int stride = kWaves * KPW;   // keys per block-load
  const int dg = lane % LPK, ks = lane / LPK;
  const int k0 = split * T.per;
  const int k1 = min(k0 + T.per, T.n);
  const int len = max(k1 - k0, 0);

  float* logit = lds;                          // [kAttnMaxKeys]
  float* red = lds + kAttnMaxKeys;             // [kWaves][256]
  float* scratch = red + kWaves * 256;         // [16]

  const size_t row0 = ((size_t)b * T.h + head) * (size_t)T.n + k0;   // first key row
  float qv[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v)
    qv[v] = T.scale * T.q[(size_t)b * T.q_ld + (size_t)slot * dh + dg * VEC + v];

  // logits
  for (int base = 0; base < len; base += stride * U) {
    float part[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * stride + wave * KPW + ks;
      float p = 0.f;
      if (j < len) {
        float kv[VEC];
        load_cols<VEC, WT>(T.K, (long long)(row0 + j) * dh + dg * VEC, kv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) p = fmaf(qv[v], kv[v], p);
      }
      part[u] = p;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      for (int off = LPK >> 1; off >= 1; off >>= 1) part[u] += __shfl_xor(part[u], off);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * stride + wave * KPW + ks;
      if (j < len && dg == 0) logit[j] = part[u];
    }
  }
  __syncthreads();
  float m = -INFINITY;
  for (int j = tid; j < len; j += kThreads) m = fmaxf(m, logit[j]);
  m = block_max(m, scratch);
  float l = 0.f;
  for (int j = tid; j < len; j += kThreads) {
    const float p = expf(logit[j] - m);
    logit[j] = p;
    l += p;
  }
  l = block_sum(l, scratch + 8);   // also orders the p writes before the reads below

  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int base = 0; base < len; base += stride * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * stride + wave * KPW + ks;
      if (j < len) {
        const float p = logit[j];
        float vv[VEC];
        load_cols<VEC, WT>(T.V, (long long)(row0 + j) * dh + dg * VEC, vv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = fmaf(p, vv[v], acc[v]);
      }
    }
  }
  for (int off = LPK; off < 64; off <<= 1)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], off);
  if (ks == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[wave * 256 + dg * VEC + v] = acc[v];
  }
  __syncthreads();
  const int w2 = dh + 2;
  float* P = T.part + (((size_t)b * cap + slot) * T.nsplit + split) * w2;
  if (tid < dh) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += red[w * 256 + tid];
    P[2 + tid] = o;
  }
  if (tid == 0) { P[0] = m; P[1] = l; }
  int* flag = reinterpret_cast<int*>(scratch + 15);
  if (!arrive_last(&T.tickets[(size_t)b * cap + slot], (uint32_t)T.nsplit, flag)) return;
  if (tid < dh) {
    const float* P0 = T.part + ((size_t)b * cap + slot) * T.nsplit * w2;
    float M = -INFINITY;
    for (int s = 0; s < T.nsplit; ++s) M = fmaxf(M, P0[(size_t)s * w2]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < T.nsplit; ++s) {
      const float ms = P0[(size_t)s * w2];
      const float wgt = (ms == -INFINITY) ? 0.f : expf(ms - M);
      L = fmaf(wgt, P0[(size_t)s * w2 + 1], L);
      O = fmaf(wgt, P0[(size_t)s * w2 + 2 + tid], O);
    }
    T.o[(size_t)b * T.o_ld + (size_t)slot * dh + tid] = O / L;
  }
}

// --------------------------------------------------------------------------- //
// top-k select and union                                                       //
// --------------------------------------------------------------------------- //

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 is mapped like +0.0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void select_row(const SelectProblem& P, int b, float* lds) {
  const int tid = threadIdx.x;
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds);      // [256]
  uint32_t* scan = hist + 256;                            // [kWaves]
  uint32_t* bcast = scan + 8;                             // [2]
  const float* s = P.scores + (size_t)b * P.ld;
  const int N = P.N;
  const int k = min(max(P.k, 0), N);

  // threshold key T and how many keys equal to T to keep (lowest indices first)
  uint32_t T, take;
  if (k == 0) {
    T = 0xffffffffu; take = 0u;
  } else if (k == N) {
    T = 0u; take = (uint32_t)N;
  } else {
    uint32_t prefix = 0u, remaining = (uint32_t)k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      __syncthreads();
      hist[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < N; j += kThreads) {
        const uint32_t key = score_key(s[j]);
        const bool match = (pass == 0) || ((key >> (shift + 8)) == (prefix >> (shift + 8)));
        if (match) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // thread t holds bin 255-t, so the inclusive scan is the count at or above that bin
      const uint32_t v = hist[255 - tid];
      uint32_t tot;
      const uint32_t inc = block_incl_scan(v, scan, &tot);
      if (v > 0u && inc >= remaining && inc - v < remaining) {
        bcast[0] = 255u - (uint32_t)tid;
        bcast[1] = inc - v;
      }
      __syncthreads();
      prefix |= bcast[0] << shift;
      remaining -= bcast[1];
    }
    T = prefix; take = remaining;
  }

  // index-ordered pass: keep key > T, and the first `take` keys == T
  uint32_t carry_eq = 0u, carry_sel = 0u;
  constexpr int E = kSelectTile / kThreads;   // 16 contiguous elements per thread
  for (int base = 0; base < N; base += kSelectTile) {
    const int j0 = base + tid * E;
    uint32_t keys[E];
    uint32_t n_eq = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = j0 + e;
      keys[e] = (j < N) ? score_key(s[j]) : 0u;
      n_eq += (j < N && keys[e] == T) ? 1u : 0u;
    }
    uint32_t tot_eq;
    uint32_t eq_before = block_incl_scan(n_eq, scan, &tot_eq) - n_eq + carry_eq;
    uint32_t selmask = 0u, n_sel = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = j0 + e;
      bool sel = false;
      if (j < N) {
        if (keys[e] > T) sel = true;
        else if (keys[e] == T) { sel = eq_before < take; ++eq_before; }
      }
      if (sel) { selmask |= 1u << e; ++n_sel; }
    }
    if (P.mode == 0) {
      uint32_t tot_sel;
      uint32_t pos = block_incl_scan(n_sel, scan, &tot_sel) - n_sel + carry_sel;
      int32_t* out = P.idx + (size_t)b * P.k;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (selmask & (1u << e)) out[pos++] = j0 + e;
      carry_sel += tot_sel;
    } else {
      // two threads fill one 32-bit word (16 elements each)
      const uint32_t other = __shfl_xor(selmask, 1);
      if ((tid & 1) == 0) {
        const int word = j0 >> 5;
        if (word < P.nwords) P.bits[(size_t)b * P.nwords + word] = selmask | (other << 16);
      }
    }
    carry_eq += tot_eq;
  }
  if (P.mode == 0 && tid == 0) P.count[b] = k;
}

__device__ __forceinline__ void select_task(const SelectTask& T, int blk, float* lds) {
  const int pi = blk / T.batch, b = blk % T.batch;
  if (pi == 0) select_row(T.p[0], b, lds);
  else select_row(T.p[1], b, lds);
}

__device__ __forceinline__ void union_problem(const UnionProblem& P, float* lds) {
  const int tid = threadIdx.x;
  uint32_t* scan = reinterpret_cast<uint32_t*>(lds);
  constexpr int E = kUnionWordsPerThread;
  uint32_t carry = 0u;
  for (int base = 0; base < P.nwords; base += kThreads * E) {
    uint32_t w[E];
    uint32_t n = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int word = base + tid * E + e;
      uint32_t x = 0u;
      if (word < P.nwords)
        for (int b = 0; b < P.batch; ++b) x |= P.bits[(size_t)b * P.nwords + word];
      w[e] = x;
      n += (uint32_t)__popc(x);
    }
    uint32_t tot;
    uint32_t pos = block_incl_scan(n, scan, &tot) - n + carry;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      uint32_t x = w[e];
      const int word = base + tid * E + e;
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1u;
        P.idx[pos++] = word * 32 + bit;
      }
    }
    carry += tot;
  }
  if (tid == 0) P.count[0] = (int32_t)carry;
}

__device__ __forceinline__ void union_task(const UnionTask& T, int blk, float* lds) {
  if (blk == 0) union_problem(T.p[0], lds);
  else union_problem(T.p[1], lds);
}

// --------------------------------------------------------------------------- //
// phase kernel                                                                 //
// --------------------------------------------------------------------------- //

template <int FLAGS, int BT>
__global__ __launch_bounds__(kThreads) void phase_kernel(PhaseArgs a) {
  extern __shared__ float lds[];
  const int blk = blockIdx.x;
  if constexpr ((FLAGS & T_ROWDOT) != 0) {
    if (blk >= a.b_rowdot && blk < a.b_rowdot + a.rowdot.blocks) {
      rowdot_task<BT>(a.rowdot, blk - a.b_rowdot, lds);
      return;
    }
  }
  if constexpr ((FLAGS & T_ATTN) != 0) {
    if (blk >= a.b_attn && blk < a.b_attn + a.attn.blocks) {
      if (a.attn.kvdt == W_BF16) attn_task<W_BF16>(a.attn, blk - a.b_attn, lds);
      else attn_task<W_F32>(a.attn, blk - a.b_attn, lds);
      return;
    }
  }
  if constexpr ((FLAGS & T_AXPY) != 0) {
    if (blk >= a.b_axpy && blk < a.b_axpy + a.axpy.blocks) {
      axpy_task<BT>(a.axpy, blk - a.b_axpy, lds);
      return;
    }
  }
  if constexpr ((FLAGS & T_SELECT) != 0) {
    if (blk >= a.b_select && blk < a.b_select + a.select.blocks) {
      select_task(a.select, blk - a.b_select, lds);
      return;
    }
  }
  if constexpr ((FLAGS & T_UNION) != 0) {
    if (blk >= a.b_union && blk < a.b_union + a.uni.blocks) {
      union_task(a.uni, blk - a.b_union, lds);
      return;
    }
  }
}

template <int FLAGS, int BT>
static int launch_t(const PhaseArgs& a, int grid, int lds_bytes, void* stream) {
  hipLaunchKernelGGL((phase_kernel<FLAGS, BT>), dim3(grid), dim3(kThreads), lds_bytes,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

template <int FLAGS>
static int launch_bt(int bt, const PhaseArgs& a, int grid, int lds_bytes, void* stream) {
  switch (bt) {
    case 1: return launch_t<FLAGS, 1>(a, grid, lds_bytes, stream);
    case 2: return launch_t<FLAGS, 2>(a, grid, lds_bytes, stream);
    default: return launch_t<FLAGS, 4>(a, grid, lds_bytes, stream);
  }
}

int launch_phase(int flags, int bt, const PhaseArgs& a, int grid, int lds_bytes, void* stream) {
  switch (flags) {
    case T_ROWDOT: return launch_bt<T_ROWDOT>(bt, a, grid, lds_bytes, stream);
    case T_AXPY: return launch_bt<T_AXPY>(bt, a, grid, lds_bytes, stream);
    case T_ATTN | T_AXPY: return launch_bt<T_ATTN | T_AXPY>(bt, a, grid, lds_bytes, stream);
    case T_AXPY | T_SELECT: return launch_bt<T_AXPY | T_SELECT>(bt, a, grid, lds_bytes, stream);
    case T_ATTN: return launch_t<T_ATTN, 1>(a, grid, lds_bytes, stream);
    case T_SELECT: return launch_t<T_SELECT, 1>(a, grid, lds_bytes, stream);
    case T_UNION: return launch_t<T_UNION, 1>(a, grid, lds_bytes, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace dv
