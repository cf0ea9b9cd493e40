// dv_kernels.hip - device code of the Deja Vu sparse decode step for gfx950.
//
// The routines are written for CDNA's 64-wide waves and 256-thread blocks:
//
//  rowdot   One wave owns one gathered row of d elements at a time and streams it
//           in 1 KiB wave-loads (16 B per lane), dotting it with the token inputs
//           staged once per block in LDS; lane partials are combined with
//           cross-lane shuffles.  Covers W1_i of Eq. (1), the d_h columns of a
//           selected W_i^Q of Eq. (2) and the predictor's first factor.
//  axpy     A block owns a (column slice x row chunk) tile: 256 bf16 columns (512 B
//           of each row) and a chunk of the gathered rows.  Each half-wave is a
//           row group that keeps 8 columns per lane in registers across every 8th
//           row; the chunk's row indices and coefficients are staged in LDS and
//           broadcast.  Row groups are summed in LDS, chunk partials are handed to
//           the last block of the slice, which adds the at most 16 chunks in a
//           fixed order: results are deterministic.  Covers W2_i scaled by ReLU(a_i)
//           in Eq. (1), W_i^O scaled by H_i(y) in Eq. (2) and the predictor's
//           second factor.
//  attn     Decode attention over the cache for one (token, selected head, key
//           split): K and V rows are loaded together and folded with a running
//           (max, sum, p.V), then the last split to finish merges the splits
//           (splitting the key axis follows the Flash-Decoding idea named on the
//           survey-notes page).
//  top-k    hist / classify (with the row's resolve in its last block), see
//           dv_internal.h.
//
// With a batch of tokens the row dots (from 2 tokens) and the row sums (from 3) run
// on the matrix cores instead (v_mfma_f32_16x16x32_bf16 over 16-row x 16-token
// tiles), so that each selected row is read once for the batch.
//
// Blocks of one launch hand values to each other only through device-coherent
// (agent-scope) atomic stores and loads plus a wait for store completion before
// the ticket: no cache writeback or invalidate is needed for that.  Values that
// a later launch reads use plain stores (a launch boundary orders them).  There are
// no floating-point atomics; only integer tickets and histograms.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <mutex>
#include <type_traits>
#include <math.h>
#include <stdint.h>

#include "dv_internal.h"

namespace dv {

// The launch descriptor travels as the kernel argument; HIP allows 4 KiB.
static_assert(sizeof(PhaseArgs) <= 4096, "PhaseArgs exceeds the kernel-argument limit");
// A row sum combining attention pieces keeps (weight, l) pairs of up to 9 head slots x
// kMaxSplit splits per token where its row groups are later reduced (the LDS of a row
// sum reserves kAxGroups * kAxSliceLanes * 8 floats per token there).

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

// 16 fp8 E4M3 codes (one 16-byte load, byte k = element k) to floats; the hardware
// conversion decodes two codes per instruction.
__device__ __forceinline__ void unpack4_fp8(uint32_t w, float* f) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}
__device__ __forceinline__ void unpack16_fp8(const uint4& x, float (&f)[16]) {
  unpack4_fp8(x.x, f);
  unpack4_fp8(x.y, f + 4);
  unpack4_fp8(x.z, f + 8);
  unpack4_fp8(x.w, f + 12);
}

// Streaming loads of weights and cache rows: each byte is read once per call, so
// the loads are marked non-temporal (they bypass reuse in the caches).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// Device-coherent accesses for values handed between blocks of one launch.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
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

// "Last block to arrive": every thread calls it after storing (st_dev) what the
// last block will read; returns true in all threads of the last arriving block.
__device__ __forceinline__ bool arrive_last(uint32_t* ticket, uint32_t expected, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's device-coherent stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (t == expected - 1u) ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

// The device's fault word: a bounded wait that gives up sets bit 0 (dv_check reports
// it), so that a launch whose blocks were not all resident at once, or whose
// producers never came, ends normally and says so instead of passing on values it
// never received.
__device__ uint32_t dv_fault;

// Waits until *ctr >= target, where other blocks of the same launch raise *ctr.
// Launches that wait are sized so all their blocks are resident at once, and a block
// only waits for work that was handed out before its own; the wait is still bounded
// (`spins` polls), so it ends even if that ever failed to hold.  Returns true in
// every thread if it gave up (after marking *fault); the caller then writes NaN
// wherever it would have used the awaited values.
// `bcast` is an LDS word of the block (free for this call) through which thread 0
// hands its outcome to the others.
__device__ __forceinline__ bool wait_ge(const uint32_t* ctr, uint32_t target, uint32_t spins,
                                        uint32_t* fault, int* bcast) {
  if (threadIdx.x == 0) {
    int gave_up = 0;
    uint32_t n = 0;
    while (__hip_atomic_load(const_cast<uint32_t*>(ctr), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (n++ >= spins) { gave_up = 1; break; }
      __builtin_amdgcn_s_sleep(8);
    }
    if (gave_up) __hip_atomic_fetch_or(fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *bcast = gave_up;
  }
  __syncthreads();
  const bool r = *bcast != 0;
  __syncthreads();
  return r;
}

// wait_ge over the ns (<= kThreads) counters ctr[(s0 + t) * kCtrStride], t < ns, polled
// together (thread t polls counter t).  `bcast`: a free LDS word, as for wait_ge.
__device__ __forceinline__ bool wait_slots_ge(const uint32_t* ctr, int s0, int ns, uint32_t target,
                                              uint32_t spins, uint32_t* fault, int* bcast) {
  if (threadIdx.x == 0) *bcast = 0;
  __syncthreads();
  if ((int)threadIdx.x < ns) {
    const uint32_t* c = ctr + (size_t)(s0 + (int)threadIdx.x) * kCtrStride;
    uint32_t n = 0;
    bool gave_up = false;
    while (__hip_atomic_load(const_cast<uint32_t*>(c), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (n++ >= spins) { gave_up = true; break; }
      __builtin_amdgcn_s_sleep(8);
    }
    if (gave_up) {
      __hip_atomic_fetch_or(fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      atomicOr(bcast, 1);
    }
  }
  __syncthreads();
  const bool r = *bcast != 0;
  __syncthreads();
  return r;
}

// Raises *ctr by one once every thread's stores of this block are complete.
__device__ __forceinline__ void signal_done(uint32_t* ctr) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// sigma of Eq. (1) applied to a row-sum coefficient: ReLU, or GeLU x Phi(x) with
// Phi(x) = (1 + erf(x / sqrt 2)) / 2 (the device library's erff).
__device__ __forceinline__ float activate(float c, int act) {
  if (act == A_RELU) return fmaxf(c, 0.f);
  if (act == A_GELU) return 0.5f * c * (1.f + erff(c * 0.70710678118654752f));
  return c;
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 is mapped like +0.0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Threshold digit from a histogram of nbins = kThreads * PT digits: thread t holds
// the counts of bins top, top-1, ..., top-PT+1 with top = nbins - 1 - t*PT, so a
// block scan in thread order counts keys from the top.  Finds the digit D holding
// the remaining-th key from the top (remaining >= 1) and the number of keys in bins
// above D; every thread receives both.
template <int PT>
__device__ __forceinline__ void find_digit(const uint32_t (&hv)[PT], uint32_t remaining,
                                           uint32_t* scratch, uint32_t* bcast, uint32_t* D,
                                           uint32_t* above) {
  const int top = kThreads * PT - 1 - (int)threadIdx.x * PT;
  uint32_t v = 0u;
#pragma unroll
  for (int j = 0; j < PT; ++j) v += hv[j];
  uint32_t tot;
  const uint32_t inc = block_incl_scan(v, scratch, &tot);
  if (v > 0u && inc >= remaining && inc - v < remaining) {
    uint32_t cum = inc - v;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      if (cum < remaining && cum + hv[j] >= remaining) {
        bcast[0] = (uint32_t)(top - j);
        bcast[1] = cum;
      }
      cum += hv[j];
    }
  }
  __syncthreads();
  *D = bcast[0];
  *above = bcast[1];
  __syncthreads();
}

// --------------------------------------------------------------------------- //
// rowdot                                                                       //
// --------------------------------------------------------------------------- //

template <int NSEG>
__device__ __forceinline__ RowdotSeg rd_seg(const RowdotTask& T, int s) {
  if constexpr (NSEG > kMaxSeg) {
    switch (s) {
      case 0: return T.seg[0];
      case 1: return T.seg[1];
      case 2: return T.seg[2];
      case 3: return T.seg[3];
      case 4: return T.seg[4];
      default: return T.seg[5];
    }
  } else {
    switch (s) {
      case 0: return T.seg[0];
      case 1: return T.seg[1];
      case 2: return T.seg[2];
      default: return T.seg[3];
    }
  }
}
// Entry s (wave-uniform) of a per-segment pointer array, by selects: fp8 row scales
// and cache stores are kept outside RowdotSeg, whose by-value selection the compiler
// keeps in registers only while the struct stays this size.
// (written as one conditional chain: a loop of selects is folded back into a dynamic
// index of the kernel argument, which the compiler then copies to scratch)
template <int NSEG, class P>
__device__ __forceinline__ P rd_pick(const P (&a)[kMaxRowdotSeg], int s) {
  if constexpr (NSEG > kMaxSeg)
    return s == 0 ? a[0] : s == 1 ? a[1] : s == 2 ? a[2] : s == 3 ? a[3] : s == 4 ? a[4] : a[5];
  else
    return s == 0 ? a[0] : s == 1 ? a[1] : s == 2 ? a[2] : a[3];
}

// float -> bfloat16 bits, rounded to nearest with ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
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
      w[u] = (v < nv) ? ld_stream(rp + v) : make_uint4(0u, 0u, 0u, 0u);
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
__device__ __forceinline__ void rowdot_fp8(const uint4* __restrict__ rp, const float* ylds, int d,
                                           int nb, int lane, float (&acc)[BT]) {
  const int nv = d >> 4;  // 16-byte vectors (16 codes) in the row
  for (int v0 = 0; v0 < nv; v0 += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 64 + lane;
      w[u] = (v < nv) ? ld_stream(rp + v) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * 64 + lane;
      if (v < nv) {
        float f[16];
        unpack16_fp8(w[u], f);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b < nb) {
            const float4* yp = reinterpret_cast<const float4*>(ylds + b * d + v * 16);
            float a = acc[b];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 yq = yp[q];
              a = fmaf(f[4 * q + 0], yq.x, a); a = fmaf(f[4 * q + 1], yq.y, a);
              a = fmaf(f[4 * q + 2], yq.z, a); a = fmaf(f[4 * q + 3], yq.w, a);
            }
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
      w[u] = (v < nv) ? ld_stream(rp + v) : make_float4(0.f, 0.f, 0.f, 0.f);
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

template <int BT, bool FP8, bool KV>
__device__ __forceinline__ void rowdot_task(const RowdotTask& T, int blk, float* lds) {
  constexpr int NSEG = KV ? kMaxRowdotSeg : kMaxSeg;
  // (the wave index as a scalar: each row's bookkeeping and id load stay in scalar
  // registers; 159 instead of 165 VGPRs at one token, and the 2- and 4-token and
  // cache-store instances fit 3 waves per SIMD instead of 2)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Counters and histograms used by later launches of the same call start at zero.
  for (int i = blk * kThreads + tid; i < T.zero_words; i += T.blocks * kThreads) T.zero_ptr[i] = 0u;

  int total_cap = 0;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) total_cap += (s < T.nseg) ? T.seg[s].cap : 0;
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
      constexpr int SU = 12;
      int i0 = tid;
      for (; i0 + (SU - 1) * kThreads < n4; i0 += kThreads * SU) {
        float4 t[SU];
#pragma unroll
        for (int u = 0; u < SU; ++u) t[u] = src[i0 + u * kThreads];
#pragma unroll
        for (int u = 0; u < SU; ++u) dst[i0 + u * kThreads] = t[u];
      }
      for (; i0 < n4; i0 += kThreads) dst[i0] = src[i0];
    }
    __syncthreads();
    for (int g = gw; g < total_cap; g += total_waves) {
      int s = 0, r = g;
#pragma unroll
      for (int i = 0; i < NSEG - 1; ++i) {
        const int c = T.seg[i].cap;
        if (s == i && r >= c) { r -= c; s = i + 1; }
      }
      const RowdotSeg S = rd_seg<NSEG>(T, s);
      const int ex = S.rows.expand;
      const int slot = (ex == 1) ? r : r / ex;
      const int e = (ex == 1) ? 0 : r - slot * ex;
      if (slot >= list_slots(S.rows)) continue;  // wave-uniform
      const int item = S.rows.idx ? S.rows.idx[slot] : slot;
      float acc[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[b] = 0.f;
      float rscale = 1.f;   // fp8 rows: the row's scale
      if ((unsigned)item < (unsigned)S.rows.items) {
        const long long row = (long long)item * ex + e;
        if (S.wdt == W_BF16) {
          const uint4* rp = reinterpret_cast<const uint4*>(
              static_cast<const uint16_t*>(S.W) + row * S.row_stride);
          rowdot_bf16<BT, 24>(rp, lds, d, nb, lane, acc);
        } else if (FP8 && S.wdt == W_FP8) {
          if constexpr (FP8) {
            const uint4* rp = reinterpret_cast<const uint4*>(
                static_cast<const uint8_t*>(S.W) + row * S.row_stride);
            rowdot_fp8<BT, 12>(rp, lds, d, nb, lane, acc);
            rscale = rd_pick<NSEG>(T.seg_scale, s)[row];
          }
        } else {
          const float4* rp = reinterpret_cast<const float4*>(
              static_cast<const float*>(S.W) + row * S.row_stride);
          rowdot_f32<BT, 8>(rp, lds, d, nb, lane, acc);
        }
      }
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[b] = FP8 ? wave_sum(acc[b]) * rscale : wave_sum(acc[b]);
      if (lane == 0) {
        void* st = nullptr;
        if constexpr (KV) st = rd_pick<NSEG>(T.seg_store, s);
        if (st) {   // the current token's k or v: stored into its cache row
          const long long o = (long long)item * T.store_ld_item + e;
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            if (b >= nb) continue;
            const long long ob = o + (long long)(b0 + b) * T.store_ld_b;
            if (T.store_dt == W_BF16) static_cast<uint16_t*>(st)[ob] = f32_to_bf16_rne(acc[b]);
            else static_cast<float*>(st)[ob] = acc[b];
          }
        } else {
#pragma unroll
          for (int b = 0; b < BT; ++b)
            if (b < nb) S.out[(size_t)(b0 + b) * S.out_ld + r] = acc[b];
        }
      }
    }
  }
}

// --------------------------------------------------------------------------- //
// rowdot on the matrix cores (a batch of tokens, bf16 rows)                    //
// --------------------------------------------------------------------------- //
//
// With B tokens the row dots are the product (B x d) . (d x rows) of Eq. (1)'s
// y W1_S (and W^Q, predictor factor A): every selected row must be read once for
// the whole batch, not once per token.  A block owns a unit of kMfmaRT tiles of
// 16 rows; its four waves take the 128-column steps of the row length in turn and
// run v_mfma_f32_16x16x32_bf16 over each: the A operand is 16 rows x 32
// columns of W (lane l holds 8 columns of row l % 16, loaded straight from HBM),
// the B operand 32 columns x 16 tokens of y.  y stays fp32 in memory; each lane
// splits its 8 values into hi = bf16(y) and mid = bf16(y - hi) and both products
// go into the fp32 accumulator, so y is represented to about 2^-17 of its
// magnitude: the predictor's scores keep an error far inside the fp32 summation
// bound the top-k comparison relies on.  The four waves' partial tiles are summed
// in LDS in wave order (deterministic) and stored like the wave-per-row path's
// results.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 8 fp32 values -> bf16 hi (nearest even) and mid = bf16(v - hi); v - hi is exact.
__device__ __forceinline__ void split8(const float4& a, const float4& b, bf16x8& hi, bf16x8& mid) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 p = {v[2 * i], v[2 * i + 1]};
    const bf16x2 h = __builtin_convertvector(p, bf16x2);
    const f32x2 hf = __builtin_convertvector(h, f32x2);
    const bf16x2 m = __builtin_convertvector(p - hf, bf16x2);
    hi[2 * i] = h[0]; hi[2 * i + 1] = h[1];
    mid[2 * i] = m[0]; mid[2 * i + 1] = m[1];
  }
}

// Segment and first logical row of row tile t (tiles of 16 rows, segments in order);
// s = -1 past the last tile.
__device__ __forceinline__ void mfma_tile(const RowdotTask& T, int t, int& s, int& r0) {
  s = -1; r0 = 0;
  int base = 0;
#pragma unroll
  for (int i = 0; i < kMaxSeg; ++i) {
    const int nt = (i < T.nseg) ? (T.seg[i].cap + kMfmaRows - 1) / kMfmaRows : 0;
    if (s < 0 && t < base + nt) { s = i; r0 = (t - base) * kMfmaRows; }
    base += nt;
  }
}

template <int NT>
__device__ __forceinline__ void rowdot_mfma_task(const RowdotTask& T, float* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = blockIdx.x * kThreads + tid; i < T.zero_words; i += gridDim.x * kThreads)
    T.zero_ptr[i] = 0u;

  int total_tiles = 0;
#pragma unroll
  for (int i = 0; i < kMaxSeg; ++i)
    total_tiles += (i < T.nseg) ? (T.seg[i].cap + kMfmaRows - 1) / kMfmaRows : 0;
  const int units = (total_tiles + kMfmaRT - 1) / kMfmaRT;
  const int d = T.d;
  const int nss = d / kMfmaCols;                 // 128-column steps (d % 128 == 0)
  const int m = lane & 15, g = lane >> 4;        // operand row / token, 8-column group
  constexpr int NACC = kMfmaRT * NT * 4;         // accumulator values per lane
  float* red = lds;                              // [kWaves][NACC][64]

  for (int tb0 = 0; tb0 < T.batch; tb0 += kMfmaRows * NT) {
    for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
      // This lane's row of each tile.  Lanes outside the list read a valid stand-in
      // row (the segment's first) instead: their products only reach output rows that
      // are not stored (or stored as 0 for an index outside [0, items)), and every
      // load stays unconditional, so the wait for a step's y leaves the next step's
      // rows in flight.  A unit with no listed row is skipped as a whole.
      const uint16_t* rp[kMfmaRT];
      bool any = false;
#pragma unroll
      for (int rt = 0; rt < kMfmaRT; ++rt) {
        int s, r0;
        mfma_tile(T, unit * kMfmaRT + rt, s, r0);
        const RowdotSeg S = rd_seg<kMaxSeg>(T, s < 0 ? 0 : s);
        rp[rt] = static_cast<const uint16_t*>(S.W) + g * 8;
        if (s >= 0) {
          const int ex = S.rows.expand;
          const int nslots = list_slots(S.rows);
          any = any || (r0 < S.cap && ((ex == 1) ? r0 : r0 / ex) < nslots);
          const int r = r0 + m;
          const int slot = (ex == 1) ? r : r / ex;
          const int e = (ex == 1) ? 0 : r - slot * ex;
          if (r < S.cap && slot < nslots) {
            const int item = S.rows.idx ? S.rows.idx[slot] : slot;
            if ((unsigned)item < (unsigned)S.rows.items)
              rp[rt] += ((long long)item * ex + e) * S.row_stride;
          }
        }
      }
      if (!any) continue;   // block-uniform
      const float* yp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = min(tb0 + nt * kMfmaRows + m, T.batch - 1);   // stand-in: last token
        yp[nt] = T.y + (size_t)n * d + g * 8;
      }
      f32x4 acc[kMfmaRT][NT];
#pragma unroll
      for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

      // The waves take the steps in turn, so a block's four waves read 512 contiguous
      // columns (1 KiB) of each of its rows at about the same time.  The rows of the
      // wave's next step are requested before the current step is computed, after
      // that step's y; the last step requests its own rows again (a cache hit).
      const int last = wave + ((nss - 1 - wave) / kWaves) * kWaves;
      uint4 w[kMfmaRT][4];
      auto load_w = [&](int ss, uint4 (&dst)[kMfmaRT][4]) {
        const int c0 = min(ss, last) * kMfmaCols;
#pragma unroll
        for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dst[rt][j] = ld_stream(reinterpret_cast<const uint4*>(rp[rt] + c0 + 32 * j));
      };
      if (wave < nss) load_w(wave, w);
      for (int ss = wave; ss < nss; ss += kWaves) {
        const int c0 = ss * kMfmaCols;
        float4 yv[NT][8];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4* q = reinterpret_cast<const float4*>(yp[nt] + c0 + 32 * j);
            yv[nt][2 * j] = q[0];
            yv[nt][2 * j + 1] = q[1];
          }
        uint4 wn[kMfmaRT][4];
        load_w(ss + kWaves, wn);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x8 hi, mid;
            split8(yv[nt][2 * j], yv[nt][2 * j + 1], hi, mid);
#pragma unroll
            for (int rt = 0; rt < kMfmaRT; ++rt) {
              const bf16x8 a = __builtin_bit_cast(bf16x8, w[rt][j]);
              acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc[rt][nt], 0, 0, 0);
              acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, mid, acc[rt][nt], 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j) w[rt][j] = wn[rt][j];
      }

      // the four waves' partial tiles, summed in wave order
      __syncthreads();
#pragma unroll
      for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            red[(wave * NACC + (rt * NT + nt) * 4 + i) * 64 + lane] = acc[rt][nt][i];
      __syncthreads();
      for (int x = tid; x < NACC * 64; x += kThreads) {
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) v += red[wv * NACC * 64 + x];
        // x = ((rt * NT + nt) * 4 + i) * 64 + ln: lane ln of the output tile holds
        // row 4 * (ln / 16) + i for token ln % 16
        const int ln = x & 63, i = (x >> 6) & 3, rtnt = x >> 8;
        const int rt = rtnt / NT, nt = rtnt - rt * NT;
        const int n = tb0 + nt * kMfmaRows + (ln & 15);
        int s, r0;
        mfma_tile(T, unit * kMfmaRT + rt, s, r0);
        if (s < 0 || n >= T.batch) continue;
        const RowdotSeg S = rd_seg<kMaxSeg>(T, s);
        const int r = r0 + 4 * (ln >> 4) + i;
        const int ex = S.rows.expand;
        const int slot = (ex == 1) ? r : r / ex;
        if (r < S.cap && slot < list_slots(S.rows)) {
          const int item = S.rows.idx ? S.rows.idx[slot] : slot;
          S.out[(size_t)n * S.out_ld + r] = ((unsigned)item < (unsigned)S.rows.items) ? v : 0.f;
        }
      }
    }
  }
}

// Matrix-core row dots with y in LDS (batch <= 32).  Loading each step's 16 tokens of
// y from L2 in every wave, as above, costs as much load throughput as the rows
// themselves (measured: 5.2 TB/s for the row stream alone, 3.2 TB/s with the y
// loads).  Here a block owns 128 rows (4 waves x 2 tiles of 16) and a part of the
// row length; its waves walk the part one 128-column step at a time together, and
// each step's y (16 tokens, split into bf16 hi / mid in MFMA B-fragment order, 8 KB)
// is staged in LDS once for the 128 rows, double-buffered.  Each wave requests the
// next step's rows and y before computing the current step (two register sets in
// turn, the last step peeled), so the rows stay in flight across the barrier.  With
// several parts per unit, each part stores its partial tile and the last part to
// finish (ticket) sums them in part order.
constexpr int kRdwRows = kWaves * kMfmaRT * kMfmaRows;   // 128 rows per unit
constexpr int kRdwFrag = 4 * 2 * 64;                     // 16-byte B fragments per step and 16 tokens
constexpr int kRdwTile = kWaves * kMfmaRT * 4 * 64;      // partial tile floats per part and 16 tokens

// NT: groups of 16 tokens (batch <= 16 NT), each with its own B fragments and accumulators
template <int NT>
__device__ __forceinline__ void rdw_task(const RowdotTask& T, float* lds) {
  constexpr int FRAG = NT * kRdwFrag;                    // fragments per LDS buffer
  constexpr int TILE = NT * kRdwTile;                    // partial tile floats per part
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  for (int i = blockIdx.x * kThreads + tid; i < T.zero_words; i += gridDim.x * kThreads)
    T.zero_ptr[i] = 0u;

  int total_tiles = 0;
#pragma unroll
  for (int i = 0; i < kMaxSeg; ++i)
    total_tiles += (i < T.nseg) ? (T.seg[i].cap + kMfmaRows - 1) / kMfmaRows : 0;
  const int units = (total_tiles + kWaves * kMfmaRT - 1) / (kWaves * kMfmaRT);
  const int d = T.d;
  const int nss = d / kMfmaCols;
  const int P = T.mfma_parts;
  const int items = units * P;
  uint4* ybuf = reinterpret_cast<uint4*>(lds);            // [2][NT][kRdwFrag]
  int* flag = reinterpret_cast<int*>(ybuf + 2 * FRAG);
  // the y fragment slot of this thread in each token group: j = tid / 64 (< 4),
  // fragment lane tid % 64
  const int yj = tid >> 6, yfl = tid & 63;

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int part = item % P;
    const int unit = item / P;
    const int s0 = part * nss / P, s1 = (part + 1) * nss / P;   // steps of this part

    const uint16_t* rp[kMfmaRT];
    bool any = false;
#pragma unroll
    for (int rt = 0; rt < kMfmaRT; ++rt) {
      int s, r0;
      mfma_tile(T, (unit * kWaves + wave) * kMfmaRT + rt, s, r0);
      const RowdotSeg S = rd_seg<kMaxSeg>(T, s < 0 ? 0 : s);
      rp[rt] = static_cast<const uint16_t*>(S.W) + g * 8;
      if (s >= 0) {
        const int ex = S.rows.expand;
        const int nslots = list_slots(S.rows);
        any = any || (r0 < S.cap && ((ex == 1) ? r0 : r0 / ex) < nslots);
        const int r = r0 + m;
        const int slot = (ex == 1) ? r : r / ex;
        const int e = (ex == 1) ? 0 : r - slot * ex;
        if (r < S.cap && slot < nslots) {
          const int it = S.rows.idx ? S.rows.idx[slot] : slot;
          if ((unsigned)it < (unsigned)S.rows.items) rp[rt] += ((long long)it * ex + e) * S.row_stride;
        }
      }
    }
    // A unit with no listed row is skipped by all its parts alike (its ticket is then
    // never needed); waves whose own tiles hold none still stage y and pass the
    // barriers (their stand-in rows reach no stored output).
    if (!__syncthreads_or(any ? 1 : 0)) continue;   // block-uniform

    auto load_w = [&](int ss, uint4 (&w)[kMfmaRT][4]) {
#pragma unroll
      for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[rt][j] = ld_stream(reinterpret_cast<const uint4*>(rp[rt] + ss * kMfmaCols + 32 * j));
    };
    // slot (group nt, j, fragment lane fl): token min(16 nt + fl % 16, batch - 1),
    // columns step * 128 + 32 j + 8 (fl / 16) .. + 8 (the columns of absent tokens
    // are never stored)
    auto load_y = [&](int ss, float4 (&yv)[NT][2]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = min(nt * kMfmaRows + (yfl & 15), T.batch - 1);
        const float4* q = reinterpret_cast<const float4*>(
            T.y + (size_t)n * d + ss * kMfmaCols + 32 * yj + (yfl >> 4) * 8);
        yv[nt][0] = q[0];
        yv[nt][1] = q[1];
      }
    };
    auto stage_y = [&](const float4 (&yv)[NT][2], int buf) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 hi, mid;
        split8(yv[nt][0], yv[nt][1], hi, mid);
        uint4* dst = ybuf + buf * FRAG + nt * kRdwFrag;
        dst[(yj * 2 + 0) * 64 + yfl] = __builtin_bit_cast(uint4, hi);
        dst[(yj * 2 + 1) * 64 + yfl] = __builtin_bit_cast(uint4, mid);
      }
    };
    f32x4 acc[kMfmaRT][NT];
#pragma unroll
    for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const uint4 (&w)[kMfmaRT][4], int buf) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4* fr = ybuf + buf * FRAG + nt * kRdwFrag;
          const bf16x8 hi = __builtin_bit_cast(bf16x8, fr[(j * 2 + 0) * 64 + lane]);
          const bf16x8 mid = __builtin_bit_cast(bf16x8, fr[(j * 2 + 1) * 64 + lane]);
#pragma unroll
          for (int rt = 0; rt < kMfmaRT; ++rt) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, w[rt][j]);
            acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc[rt][nt], 0, 0, 0);
            acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, mid, acc[rt][nt], 0, 0, 0);
          }
        }
    };
    // one step with the next one's y and rows requested first (issue order y, rows:
    // the load counter is in order, so waiting for y does not wait for the rows)
    auto step = [&](int ss, const uint4 (&cur)[kMfmaRT][4], uint4 (&nxt)[kMfmaRT][4]) {
      float4 yv[NT][2];
      load_y(ss + 1, yv);
      __builtin_amdgcn_sched_barrier(0);
      load_w(ss + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      compute(cur, (ss - s0) & 1);
      __builtin_amdgcn_sched_barrier(0);
      stage_y(yv, (ss + 1 - s0) & 1);
      __syncthreads();
    };

    uint4 wa[kMfmaRT][4], wb[kMfmaRT][4];
    {
      float4 yv[NT][2];
      load_y(s0, yv);
      __builtin_amdgcn_sched_barrier(0);
      load_w(s0, wa);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();                          // the previous item's last reads of ybuf
      stage_y(yv, 0);
      __syncthreads();
    }
    int ss = s0;
    for (; ss + 2 < s1; ss += 2) {
      step(ss, wa, wb);
      step(ss + 1, wb, wa);
    }
    if (ss + 1 < s1) {                          // two steps left: the last one peeled
      step(ss, wa, wb);
      compute(wb, (ss + 1 - s0) & 1);
    } else {                                    // one step left
      compute(wa, (ss - s0) & 1);
    }

    // the wave's outputs: lane ln of tile rt, group nt holds rows 4 (ln / 16) + i,
    // token 16 nt + ln % 16
    float v[kMfmaRT][NT][4];
#pragma unroll
    for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[rt][nt][i] = acc[rt][nt][i];
    if (P > 1) {
      float* base = T.mfma_partial + (size_t)unit * P * TILE;
      const int off = (wave * kMfmaRT * NT * 4) * 64 + lane;
#pragma unroll
      for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st_dev(&base[(size_t)part * TILE + off + ((rt * NT + nt) * 4 + i) * 64], v[rt][nt][i]);
      if (!arrive_last(&T.mfma_tickets[unit], (uint32_t)P, flag)) continue;   // block-uniform
#pragma unroll
      for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[rt][nt][i] = 0.f;
      for (int p = 0; p < P; ++p) {             // part order; 8 NT loads in flight per part
        float t[kMfmaRT][NT][4];
#pragma unroll
        for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              t[rt][nt][i] = ld_dev(&base[(size_t)p * TILE + off + ((rt * NT + nt) * 4 + i) * 64]);
#pragma unroll
        for (int rt = 0; rt < kMfmaRT; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[rt][nt][i] += t[rt][nt][i];
      }
    }
    if (!any) continue;
#pragma unroll
    for (int rt = 0; rt < kMfmaRT; ++rt) {
      int s, r0;
      mfma_tile(T, (unit * kWaves + wave) * kMfmaRT + rt, s, r0);
      if (s < 0) continue;
      const RowdotSeg S = rd_seg<kMaxSeg>(T, s);
      const int ex = S.rows.expand;
      const int nslots = list_slots(S.rows);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = nt * kMfmaRows + m;
        if (n >= T.batch) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r0 + 4 * g + i;
          const int slot = (ex == 1) ? r : r / ex;
          if (r < S.cap && slot < nslots) {
            const int it = S.rows.idx ? S.rows.idx[slot] : slot;
            S.out[(size_t)n * S.out_ld + r] = ((unsigned)it < (unsigned)S.rows.items) ? v[rt][nt][i] : 0.f;
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------------------- //
// axpy                                                                         //
// --------------------------------------------------------------------------- //

constexpr int kAxpyTile = kAxpyTileRows;

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
    unpack8(ld_stream(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + off)), f);
#pragma unroll
    for (int v = 0; v < 8; ++v) w[v] = f[v];
  } else if constexpr (WT == W_FP8 && VEC == 16) {
    unpack16_fp8(ld_stream(reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(W) + off)), w);
  } else if constexpr (WT == W_F32 && VEC == 4) {
    const float4 x = ld_stream(reinterpret_cast<const float4*>(static_cast<const float*>(W) + off));
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (WT == W_BF16) {
    w[0] = __uint_as_float((uint32_t)(static_cast<const uint16_t*>(W)[off]) << 16);
  } else {
    w[0] = static_cast<const float*>(W)[off];
  }
}

// Adds the top-digit of each active thread's score to an LDS histogram, then the
// non-zero bins to the device histogram `gh`.  All threads of the block call.
__device__ __forceinline__ void hist_flush_one(float score, bool active, uint32_t* lh, uint32_t* gh) {
  const int tid = threadIdx.x;
  __syncthreads();
  for (int i = tid; i < kHistBins; i += kThreads) lh[i] = 0u;
  __syncthreads();
  if (active) atomicAdd(&lh[score_key(score) >> kTopShift], 1u);
  __syncthreads();
  for (int i = tid; i < kHistBins; i += kThreads) {
    const uint32_t c = lh[i];
    if (c) __hip_atomic_fetch_add(&gh[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// U rows of one fp8 row group: the 16-byte loads (16 columns per lane) are issued
// together and stay packed until each row is decoded and accumulated, so the row
// group keeps U rows in flight within the register budget.  `at(row)` gives a row's
// 16 bytes for this lane.
template <int BT, int U, class At>
__device__ __forceinline__ void fp8_rows(const int* lrow, const float* lcoef, int i0, int tn,
                                         At at, float (&acc)[BT][16]) {
  uint4 wr[U];
  float c[U][BT];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = i0 + u * kAxGroups;
    const int row = (i < tn) ? lrow[i] : -1;
    wr[u] = (row >= 0) ? ld_stream(at(row)) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int b = 0; b < BT; ++b) c[u][b] = (i < tn) ? lcoef[b * kAxpyTile + i] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float f[16];
    unpack16_fp8(wr[u], f);
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[b][v] = fmaf(c[u][b], f[v], acc[b][v]);
  }
}

// The same for bf16 rows (8 columns per lane): packed 16-byte loads, unpacked one row
// at a time, so a row group keeps twice the rows in flight that unpacked loads would
// allow in the same registers.
template <int BT, int U, class At>
__device__ __forceinline__ void bf16_rows(const int* lrow, const float* lcoef, int i0, int tn,
                                          At at, float (&acc)[BT][8]) {
  uint4 wr[U];
  float c[U][BT];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = i0 + u * kAxGroups;
    const int row = (i < tn) ? lrow[i] : -1;
    wr[u] = (row >= 0) ? ld_stream(at(row)) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int b = 0; b < BT; ++b) c[u][b] = (i < tn) ? lcoef[b * kAxpyTile + i] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float f[8];
    unpack8(wr[u], f);
#pragma unroll
    for (int b = 0; b < BT; ++b)
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[b][v] = fmaf(c[u][b], f[v], acc[b][v]);
  }
}

// Rows [r0, r1) of chunk c of C chunks over n rows.  With skew > 0 earlier chunks take
// more rows (weight skew (C-1-c) + 8 (C-1)): their blocks come first in block order,
// and on a CU the older waves issue first, so they stream faster than the blocks
// dispatched after them.
__device__ __forceinline__ void chunk_range(int c, int C, int n, int skew, int& r0, int& r1) {
  if (skew == 0 || C <= 1) {
    const int per = (n + C - 1) / C;
    r0 = min(c * per, n);
    r1 = min(r0 + per, n);
    return;
  }
  auto W = [&](long long x) {
    return (long long)skew * (x * (C - 1) - x * (x - 1) / 2) + 8ll * (C - 1) * x;
  };
  const long long tot = W(C);
  r0 = (int)((long long)n * W(c) / tot);
  r1 = (int)((long long)n * W(c + 1) / tot);
}

// One block: a slice of kAxSliceLanes*VEC output columns and a chunk of the row list.
template <int BT, int VEC, int WT, bool WAIT>
__device__ __forceinline__ void axpy_block(const AxpySeg& S, const float* sc1, const float* sc2,
                                           int lb, int batch, float* lds,
                                           const AxpyTask* task = nullptr) {
  // rows in flight per row group: packed bf16 loads hold more in the registers that 4
  // unpacked ones take; fp8 rows (16 columns a lane, 16 sums per token) keep 4 at the
  // 64-register cap and take more in the waiting launch, which runs without it
  constexpr bool PACKED = WT == W_BF16 && VEC == 8;
  constexpr int U = PACKED ? kAxPackedU : (WT == W_FP8 && WAIT) ? kAxFp8WaitU : 4;
  constexpr int SW = kAxSliceLanes * VEC;    // columns per slice
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave * 2 + (lane >> 5);
  const int hl = lane & 31;
  const int slice = lb % S.nslices;
  const int rest = lb / S.nslices;
  const int chunk = rest % S.nchunks;
  const int bti = rest / S.nchunks;
  const int b0 = bti * BT;
  const int nb = min(BT, batch - b0);
  const int col0 = slice * SW + hl * VEC;
  const bool active = col0 < S.ncols;

  int* lrow = reinterpret_cast<int*>(lds);               // [kAxpyTile] row or -1 (see below)
  float* lcoef = lds + kAxpyTile;                        // [BT][kAxpyTile]
  float* red = lds + kAxpyTile * (1 + BT);               // [kAxGroups][BT][SW]

  float acc[BT][VEC];
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[b][v] = 0.f;

  if constexpr (!WAIT) {
    // The rows of both sources form one list, the first source's rows first; chunk
    // c takes a contiguous share of it.  lrow marks second-source rows with bit 30.
    const int nrows_a = list_slots(S.rows) * S.rows.expand;
    const int nrows = nrows_a + (S.W2 ? list_slots(S.rows2) * S.rows2.expand : 0);
    int r0, r1;
    chunk_range(chunk, S.nchunks, nrows, task ? task->skew : 0, r0, r1);

    for (int t0 = r0; t0 < r1; t0 += kAxpyTile) {
      const int tn = min(kAxpyTile, r1 - t0);
      __syncthreads();
      for (int i = tid; i < tn; i += kThreads) {
        const bool second = t0 + i >= nrows_a;
        const int rr = second ? t0 + i - nrows_a : t0 + i;
        const RowList& L = second ? S.rows2 : S.rows;
        const int ex = L.expand;
        const int slot = (ex == 1) ? rr : rr / ex;
        const int e = (ex == 1) ? 0 : rr - slot * ex;
        const int item = L.idx ? L.idx[slot] : slot;
        const bool ok = (unsigned)item < (unsigned)L.items;
        lrow[i] = ok ? ((item * ex + e) | (second ? (1 << 30) : 0)) : -1;
        const float* cf = second ? S.coef2 : S.coef;
        const int cld = second ? S.coef2_ld : S.coef_ld;
        const int rl = second ? S.act2 : S.act;
        const float* sc = second ? sc2 : sc1;
  #pragma unroll
        for (int b = 0; b < BT; ++b) {
          float c = 0.f;
          if (ok && b < nb) {
            c = cf[(size_t)(b0 + b) * cld + rr];
            c = activate(c, rl);
            if constexpr (WT == W_FP8) c *= sc[item * ex + e];   // row scale folded in
          }
          lcoef[b * kAxpyTile + i] = c;
        }
      }
      __syncthreads();
      if (active) {
        for (int i0 = grp; i0 < tn; i0 += kAxGroups * U) {
          if constexpr (WT == W_FP8) {
            fp8_rows<BT, U>(lrow, lcoef, i0, tn, [&](int row) {
              const void* W = (row & (1 << 30)) ? S.W2 : S.W;
              return reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(W) +
                  (long long)(row & ((1 << 30) - 1)) * S.row_stride + col0);
            }, acc);
            continue;
          } else if constexpr (PACKED) {
            bf16_rows<BT, U>(lrow, lcoef, i0, tn, [&](int row) {
              const void* W = (row & (1 << 30)) ? S.W2 : S.W;
              return reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) +
                  (long long)(row & ((1 << 30) - 1)) * S.row_stride + col0);
            }, acc);
            continue;
          }
          float w[U][VEC];
          float c[U][BT];
  #pragma unroll
          for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kAxGroups;
            const int row = (i < tn) ? lrow[i] : -1;
            if (row >= 0) {
              const void* W = (row & (1 << 30)) ? S.W2 : S.W;
              load_cols<VEC, WT>(W, (long long)(row & ((1 << 30) - 1)) * S.row_stride + col0, w[u]);
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
  } else {
    // Chunk c takes its share of the first source's rows, then its share of the
    // second's; a block may wait between the two for coefficients of the second source
    // produced in the same launch.
    const int n1 = list_slots(S.rows) * S.rows.expand;
    const int n2 = S.W2 ? list_slots(S.rows2) * S.rows2.expand : 0;
    // the chunk's contiguous share [r0, r1) of nr rows
    auto share = [&](int nr, int& r0, int& r1) { chunk_range(chunk, S.nchunks, nr, 0, r0, r1); };
    int r0 = 0, r1 = 0, q0 = 0, q1 = 0;
    if (task->c2 > 0) {
      // separate chunks for the two sources; the first source's come first in block
      // order, so their blocks are dispatched first and the second source's blocks wait
      // for their coefficients without holding back the first source's stream
      const int c1 = S.nchunks - task->c2;
      if (chunk < c1) chunk_range(chunk, c1, n1, 0, r0, r1);
      else chunk_range(chunk - c1, task->c2, n2, 0, q0, q1);
    } else {
      share(n1, r0, r1);
      share(n2, q0, q1);
    }
    const int m1 = r1 - r0, m2 = q1 - q0;

    if constexpr (PACKED) {
      const int ex2 = S.W2 ? S.rows2.expand : 1;
      if (S.wait_ctr && m1 + m2 <= kAxpyTile &&
          (m2 == 0 || (q1 - 1) / ex2 - q0 / ex2 < kThreads)) {
        // Both shares fit one tile: the row ids of both and the first source's
        // coefficients are staged together; the first step of second-source rows is
        // loaded before its coefficients are ready, then the block waits for the slots
        // those rows belong to (all at once) and stages their coefficients.
        const void* const W1 = S.W;
        const void* const W2 = S.W2;
        __syncthreads();
        for (int i = tid; i < m1 + m2; i += kThreads) {
          const bool second = i >= m1;
          const RowList& L = second ? S.rows2 : S.rows;
          const int rr = second ? q0 + i - m1 : r0 + i;
          const int ex = L.expand;
          const int slot = (ex == 1) ? rr : rr / ex;
          const int e = (ex == 1) ? 0 : rr - slot * ex;
          const int item = L.idx ? L.idx[slot] : slot;
          const bool ok = (unsigned)item < (unsigned)L.items;
          lrow[i] = ok ? item * ex + e : -1;
          if (!second) {
#pragma unroll
            for (int b = 0; b < BT; ++b)
              lcoef[b * kAxpyTile + i] =
                  (ok && b < nb) ? activate(S.coef[(size_t)(b0 + b) * S.coef_ld + rr], S.act) : 0.f;
          }
        }
        __syncthreads();
        auto at1 = [&](int row) {
          return reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W1) +
                                                (long long)row * S.row_stride + col0);
        };
        auto at2 = [&](int row) {
          return reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W2) +
                                                (long long)row * S.row_stride + col0);
        };
        if (active)
          for (int i0 = grp; i0 < m1; i0 += kAxGroups * U) bf16_rows<BT, U>(lrow, lcoef, i0, m1, at1, acc);
        if (m2 > 0) {
          constexpr int UP = kAxPrefetchU < U ? kAxPrefetchU : U;   // rows loaded early
          uint4 wpre[UP];
#pragma unroll
          for (int u = 0; u < UP; ++u) {
            const int i = grp + u * kAxGroups;
            const int row = (active && i < m2) ? lrow[m1 + i] : -1;
            wpre[u] = (row >= 0) ? ld_stream(at2(row)) : make_uint4(0u, 0u, 0u, 0u);
          }
          const int s0 = q0 / ex2, s1 = (q1 - 1) / ex2;
          const bool gave_up = wait_slots_ge(S.wait_ctr, s0, s1 - s0 + 1, S.wait_target,
                                             task->spins, task->fault, reinterpret_cast<int*>(red));
          if (task->part2) {
            // o from the key splits' softmax pieces (max m, sum l, p.V): the (m, l) of
            // every (token, slot, split) of the share go to LDS, each row's p.V pieces
            // are fetched by its thread; o = sum_s w_s pV_s / sum_s w_s l_s with
            // w_s = exp(m_s - max m), summed in split order
            const int ns = task->nsplit2, w2 = ex2 + 2, cap2 = S.rows2.host_count;
            float* pm = red + 64;                            // [BT][slots][ns]
            float* pl = pm + BT * (s1 - s0 + 1) * ns;
            const int npc = nb * (s1 - s0 + 1) * ns;
            for (int t = tid; t < npc; t += kThreads) {
              const int sp = t % ns, r = t / ns;
              const int ls = r % (s1 - s0 + 1), b = r / (s1 - s0 + 1);
              const float* P = task->part2 +
                  (((size_t)(b0 + b) * cap2 + s0 + ls) * ns + sp) * w2;
              pm[t] = ld_dev(&P[0]);
              pl[t] = ld_dev(&P[1]);
            }
            __syncthreads();
            for (int i = tid; i < m2; i += kThreads) {
              const int rr = q0 + i, slot = rr / ex2, e = rr - slot * ex2;
#pragma unroll
              for (int b = 0; b < BT; ++b) {
                float c = 0.f;
                if (lrow[m1 + i] >= 0 && b < nb) {
                  const float* sm_ = pm + (b * (s1 - s0 + 1) + slot - s0) * ns;
                  const float* sl_ = pl + (b * (s1 - s0 + 1) + slot - s0) * ns;
                  const float* P0 = task->part2 + (((size_t)(b0 + b) * cap2 + slot) * ns) * w2;
                  float MM = -INFINITY;
                  for (int sp = 0; sp < ns; ++sp) MM = fmaxf(MM, sm_[sp]);
                  float LL = 0.f, OO = 0.f;
                  constexpr int UB = 8;
                  for (int sp0 = 0; sp0 < ns; sp0 += UB) {
                    float ov[UB];
#pragma unroll
                    for (int u = 0; u < UB; ++u)
                      ov[u] = ld_dev(&P0[(size_t)min(sp0 + u, ns - 1) * w2 + 2 + e]);
#pragma unroll
                    for (int u = 0; u < UB; ++u) {
                      if (sp0 + u < ns) {
                        const float ms = sm_[sp0 + u];
                        const float wgt = (ms == -INFINITY) ? 0.f : expf(ms - MM);
                        LL = fmaf(wgt, sl_[sp0 + u], LL);
                        OO = fmaf(wgt, ov[u], OO);
                      }
                    }
                  }
                  c = activate(OO / LL, S.act2);
                  if (gave_up) c = __builtin_nanf("");
                }
                lcoef[b * kAxpyTile + m1 + i] = c;
              }
            }
          } else {
            for (int i = tid; i < m2; i += kThreads) {
#pragma unroll
              for (int b = 0; b < BT; ++b) {
                float c = 0.f;
                if (lrow[m1 + i] >= 0 && b < nb) {
                  c = activate(ld_dev(&S.coef2[(size_t)(b0 + b) * S.coef2_ld + q0 + i]), S.act2);
                  if (gave_up) c = __builtin_nanf("");
                }
                lcoef[b * kAxpyTile + m1 + i] = c;
              }
            }
          }
          __syncthreads();
          if (active) {
#pragma unroll
            for (int u = 0; u < UP; ++u) {
              const int i = grp + u * kAxGroups;
              if (i < m2) {
                float f[8];
                unpack8(wpre[u], f);
#pragma unroll
                for (int b = 0; b < BT; ++b) {
                  const float c = lcoef[b * kAxpyTile + m1 + i];
#pragma unroll
                  for (int v = 0; v < 8; ++v) acc[b][v] = fmaf(c, f[v], acc[b][v]);
                }
              }
            }
            for (int i0 = grp + kAxGroups * UP; i0 < m2; i0 += kAxGroups * U)
              bf16_rows<BT, U>(lrow + m1, lcoef + m1, i0, m2, at2, acc);
          }
        }
        goto reduce;
      }
    }

    // one source's share of rows: coefficients staged in LDS a tile at a time, then the
    // row slices streamed by the row groups
    auto rows_of = [&](const RowList& L, const void* W, const float* cf, int cld, int rl,
                       const float* sc, bool coherent, int r0, int r1, bool poison) {
      const int ex = L.expand;
      for (int t0 = r0; t0 < r1; t0 += kAxpyTile) {
        const int tn = min(kAxpyTile, r1 - t0);
        __syncthreads();
        for (int i = tid; i < tn; i += kThreads) {
          const int rr = t0 + i;
          const int slot = (ex == 1) ? rr : rr / ex;
          const int e = (ex == 1) ? 0 : rr - slot * ex;
          const int item = L.idx ? L.idx[slot] : slot;
          const bool ok = (unsigned)item < (unsigned)L.items;
          lrow[i] = ok ? item * ex + e : -1;
  #pragma unroll
          for (int b = 0; b < BT; ++b) {
            float c = 0.f;
            if (ok && b < nb) {
              const float* cp = &cf[(size_t)(b0 + b) * cld + rr];
              c = coherent ? ld_dev(cp) : *cp;
              c = activate(c, rl);
              if constexpr (WT == W_FP8) c *= sc[item * ex + e];
              if (poison) c = __builtin_nanf("");
            }
            lcoef[b * kAxpyTile + i] = c;
          }
        }
        __syncthreads();
        if (active) {
          for (int i0 = grp; i0 < tn; i0 += kAxGroups * U) {
            if constexpr (WT == W_FP8) {
              fp8_rows<BT, U>(lrow, lcoef, i0, tn, [&](int row) {
                return reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(W) +
                                                      (long long)row * S.row_stride + col0);
              }, acc);
              continue;
            } else if constexpr (PACKED) {
              bf16_rows<BT, U>(lrow, lcoef, i0, tn, [&](int row) {
                return reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) +
                                                      (long long)row * S.row_stride + col0);
              }, acc);
              continue;
            }
            float w[U][VEC];
            float c[U][BT];
  #pragma unroll
            for (int u = 0; u < U; ++u) {
              const int i = i0 + u * kAxGroups;
              const int row = (i < tn) ? lrow[i] : -1;
              if (row >= 0) {
                load_cols<VEC, WT>(W, (long long)row * S.row_stride + col0, w[u]);
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
    };
    rows_of(S.rows, S.W, S.coef, S.coef_ld, S.act, sc1, false, r0, r1, false);
    if (!S.wait_ctr) {
      rows_of(S.rows2, S.W2, S.coef2, S.coef2_ld, S.act2, sc2, false, q0, q1, false);
    } else {
      // coefficients of the second source written in this launch, one slot at a time:
      // wait for that slot's counter, then read its coefficients coherently
      const int ex = S.rows2.expand;
      for (int a = q0; a < q1;) {
        const int slot = a / ex;
        const int e = min(q1, (slot + 1) * ex);
        const bool gave_up = wait_ge(S.wait_ctr + (size_t)slot * kCtrStride, S.wait_target,
                                     task->spins, task->fault, reinterpret_cast<int*>(lds));
        // (coefficients left as attention pieces are combined only on the one-tile
        // path, which the launch is planned to take: reaching here with them is a
        // planning error, and the outputs are NaN)
        rows_of(S.rows2, S.W2, S.coef2, S.coef2_ld, S.act2, sc2, true, a, e,
                gave_up || task->part2 != nullptr);
        a = e;
      }
    }
  }

reduce:
  // sum the row groups in order 0..7
  __syncthreads();
#pragma unroll
  for (int b = 0; b < BT; ++b)
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[(grp * BT + b) * SW + hl * VEC + v] = acc[b][v];
  __syncthreads();
  // each thread finalises CPT output columns of the slice (2 for 16-column fp8 lanes)
  constexpr int CPT = (SW + kThreads - 1) / kThreads;
  const size_t ncols = (size_t)S.ncols;
  int colv[CPT];
  bool cactv[CPT];
  float part[CPT][BT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int cc = tid + j * kThreads;
    colv[j] = slice * SW + cc;
    cactv[j] = cc < SW && colv[j] < S.ncols;
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      float t = 0.f;
      if (cactv[j]) {
#pragma unroll
        for (int g = 0; g < kAxGroups; ++g) t += red[(g * BT + b) * SW + cc];
      }
      part[j][b] = t;
    }
  }

  if (S.nchunks > 1) {
    float* P = S.partial + ((size_t)(bti * S.nchunks + chunk) * BT) * ncols;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      if (cactv[j]) {
#pragma unroll
        for (int b = 0; b < BT; ++b)
          if (b < nb) st_dev(&P[b * ncols + colv[j]], part[j][b]);
      }
    }
    int* flag = reinterpret_cast<int*>(lds);
    if (!arrive_last(&S.tickets[bti * S.nslices + slice], (uint32_t)S.nchunks, flag)) return;
    const float* P0 = S.partial + (size_t)bti * S.nchunks * BT * ncols;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        if (b < nb && cactv[j]) {
          float v[kMaxChunks];
#pragma unroll
          for (int c = 0; c < kMaxChunks; ++c)
            v[c] = (c < S.nchunks) ? ld_dev(&P0[((size_t)c * BT + b) * ncols + colv[j]]) : 0.f;
          float t = 0.f;
#pragma unroll
          for (int c = 0; c < kMaxChunks; ++c) t += v[c];
          part[j][b] = t;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      if (b < nb && cactv[j]) {
        const size_t bo = (size_t)(b0 + b);
        const int col = colv[j];
        float sum = part[j][b];
        if (S.add1) sum = S.add1[bo * S.add_ld + col] + sum;
        if (S.add0) sum = S.add0[bo * S.add_ld + col] + sum;
        float* o = S.out + bo * S.out_ld + col;
        if (S.accumulate) sum = *o + sum;
        *o = sum;
        part[j][b] = sum;
      }
    }
  }
  if constexpr (CPT == 1) {
    if (S.hist) {
      uint32_t* lh = reinterpret_cast<uint32_t*>(lds) + 16;
#pragma unroll
      for (int b = 0; b < BT; ++b)
        if (b < nb) hist_flush_one(part[0][b], cactv[0], lh, S.hist + (size_t)(b0 + b) * kHistBins);
    }
  }
}

// --------------------------------------------------------------------------- //
// axpy on the matrix cores (a batch of tokens, bf16 rows)                      //
// --------------------------------------------------------------------------- //
//
// out[b][col] = sum_s c[b][s] R[row(s)][col] contracts over the row index, while a
// row is contiguous along col.  The MFMA operand wants the contracted index along
// a lane's eight values, so each lane loads an 8 x 8 block (16 bytes from each of
// 8 consecutive rows of the list, at the same 8 columns) and regroups it in
// registers into eight column vectors of 8 rows.  Vector j of lane l is the A
// operand row l % 16 of MFMA j: MFMA j (v_mfma_f32_16x16x32_bf16) covers the 16
// columns col0 + 8 m + j (m < 16) against 32 rows and 16 tokens.  Eight MFMAs
// cover a 128-column slice.  Coefficients (fp32) are split into bf16 hi + mid like
// the row dots' y.  A block owns a (128-column slice x row chunk x token tile):
// its four waves take 32-row groups in turn and are summed in LDS in wave order;
// chunk partials go to the last block of the slice (tickets), which sums them in
// chunk order and applies the epilogue: deterministic, like the wave path.
constexpr int kAxmCoefLd = kAxmTile + 4; // padded row of the coefficient tile
constexpr int kAxmRedLd = kMfmaCols + 1; // padded row of the wave sums

// Low / high bf16 halves of two words packed into one word (row a low, row b high).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int NT>
__device__ __forceinline__ void axpy_mfma_block(const AxpySeg& S, int lb, int batch, int skew,
                                                float* lds) {
  constexpr int TB = kMfmaRows * NT;       // tokens per block tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int m = lane & 15, g = lane >> 4;
  const int slice = lb % S.nslices;
  const int rest = lb / S.nslices;
  const int chunk = rest % S.nchunks;
  const int bti = rest / S.nchunks;
  const int b0 = bti * TB;
  const int nb = min(TB, batch - b0);
  const int col0 = slice * kMfmaCols;

  int* lrow = reinterpret_cast<int*>(lds);               // [kAxmTile] row or -1
  float* lcoef = lds + kAxmTile;                         // [TB][kAxmCoefLd]
  float* red = lcoef + TB * kAxmCoefLd;                  // [TB][kAxmRedLd]

  f32x4 acc[NT][8];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[nt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The rows of both sources form one list (first source first); chunk c takes a
  // contiguous share; lrow marks second-source rows with bit 30.
  const int nrows_a = list_slots(S.rows) * S.rows.expand;
  const int nrows = nrows_a + (S.W2 ? list_slots(S.rows2) * S.rows2.expand : 0);
  int r0, r1;
  chunk_range(chunk, S.nchunks, nrows, skew, r0, r1);

  for (int t0 = r0; t0 < r1; t0 += kAxmTile) {
    const int tn = min(kAxmTile, r1 - t0);
    __syncthreads();
    for (int i = tid; i < kAxmTile; i += kThreads) {
      int rowv = -1;
      bool ok = false, second = false;
      int rr = 0;
      if (i < tn) {
        second = t0 + i >= nrows_a;
        rr = second ? t0 + i - nrows_a : t0 + i;
        const RowList& L = second ? S.rows2 : S.rows;
        const int ex = L.expand;
        const int slot = (ex == 1) ? rr : rr / ex;
        const int e = (ex == 1) ? 0 : rr - slot * ex;
        const int item = L.idx ? L.idx[slot] : slot;
        ok = (unsigned)item < (unsigned)L.items;
        if (ok) rowv = (item * ex + e) | (second ? (1 << 30) : 0);
      }
      lrow[i] = rowv;
      const float* cf = second ? S.coef2 : S.coef;
      const int cld = second ? S.coef2_ld : S.coef_ld;
      const int rl = second ? S.act2 : S.act;
      // all TB coefficient loads of the row are issued before any is used (one round
      // trip per tile rather than one per few tokens)
      float cv[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b)
        cv[b] = (ok && b < nb) ? cf[(size_t)(b0 + min(b, nb - 1)) * cld + rr] : 0.f;
#pragma unroll
      for (int b = 0; b < TB; ++b)
        lcoef[b * kAxmCoefLd + i] = (ok && b < nb) ? activate(cv[b], rl) : 0.f;
    }
    __syncthreads();
    // 16 bytes of each of the rows q + 8 g + i, i < 8, at columns col0 + 8 m.  Rows
    // outside the list load a stand-in (row 0 of the first source) and are zeroed,
    // so every load is unconditional and the next group's rows stay in flight while
    // this group is computed.
    auto load_rows = [&](int q, uint4 (&dst)[8], uint32_t& valid) {
      valid = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = lrow[q + 8 * g + i];
        const int rr = row < 0 ? 0 : row;
        const void* W = (rr & (1 << 30)) ? S.W2 : S.W;
        dst[i] = ld_stream(reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(W) + (long long)(rr & ((1 << 30) - 1)) * S.row_stride +
            col0 + 8 * m));
        valid |= (row >= 0 ? 1u : 0u) << i;
      }
    };
    auto group = [&](int q, const uint4 (&w)[8], uint32_t valid) {
      bf16x8 chi[NT], cmid[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float4* cp = reinterpret_cast<const float4*>(lcoef + (nt * kMfmaRows + m) * kAxmCoefLd +
                                                           q + 8 * g);
        split8(cp[0], cp[1], chi[nt], cmid[nt]);
      }
      // column vectors: element i of vector j = row 8 g + i, column col0 + 8 m + j;
      // word x of row i, zero for rows outside the list, is taken where it is used
      auto word = [&](int i, int x) -> uint32_t {
        const uint32_t v = x == 0 ? w[i].x : x == 1 ? w[i].y : x == 2 ? w[i].z : w[i].w;
        return ((valid >> i) & 1u) ? v : 0u;
      };
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t a[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo = word(2 * p, j >> 1), hi = word(2 * p + 1, j >> 1);
          a[p] = (j & 1) ? pack_hi(lo, hi) : pack_lo(lo, hi);
        }
        const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(a[0], a[1], a[2], a[3]));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, chi[nt], acc[nt][j], 0, 0, 0);
          acc[nt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, cmid[nt], acc[nt][j], 0, 0, 0);
        }
      }
    };
    // this wave's 32-row groups of the tile, two register sets in turn (no copy waits
    // for the next group's rows); past the last group the "next" rows repeat it
    int q = wave * 32;
    if (q < tn) {
      uint4 wa[8], wb[8];
      uint32_t va, vb;
      load_rows(q, wa, va);
      // (the scheduling barriers keep each group's loads ahead of the previous
      // group's arithmetic, so the wait for one set does not cover the other)
      for (;;) {
        int qn = q + kWaves * 32;
        __builtin_amdgcn_sched_barrier(0);
        load_rows(qn < tn ? qn : q, wb, vb);
        __builtin_amdgcn_sched_barrier(0);
        group(q, wa, va);
        if (qn >= tn) break;
        q = qn;
        qn = q + kWaves * 32;
        __builtin_amdgcn_sched_barrier(0);
        load_rows(qn < tn ? qn : q, wa, va);
        __builtin_amdgcn_sched_barrier(0);
        group(q, wb, vb);
        if (qn >= tn) break;
        q = qn;
      }
    }
  }

  // Sum the waves in wave order.  Lane l of MFMA j holds, for token l % 16, the
  // columns col0 + 8 (4 (l / 16) + i) + j, i < 4.
  for (int wv = 0; wv < kWaves; ++wv) {
    __syncthreads();
    if (wave == wv) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float* rp = &red[(nt * kMfmaRows + m) * kAxmRedLd + 8 * (4 * g + i) + j];
            *rp = (wv == 0) ? acc[nt][j][i] : *rp + acc[nt][j][i];
          }
    }
  }
  __syncthreads();

  // each thread finalises column tid % 128 of tokens 2 it + tid / 128
  constexpr int PER = TB * kMfmaCols / kThreads;
  const int cc = tid & (kMfmaCols - 1), th = tid >> 7;
  const size_t ncols = (size_t)S.ncols;
  const int col = col0 + cc;
  float part[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) part[it] = red[(2 * it + th) * kAxmRedLd + cc];

  if (S.nchunks > 1) {
    float* P = S.partial + ((size_t)(bti * S.nchunks + chunk) * TB) * ncols;
#pragma unroll
    for (int it = 0; it < PER; ++it)
      if (2 * it + th < nb) st_dev(&P[(2 * it + th) * ncols + col], part[it]);
    int* flag = reinterpret_cast<int*>(lds);
    if (!arrive_last(&S.tickets[bti * S.nslices + slice], (uint32_t)S.nchunks, flag)) return;
    const float* P0 = S.partial + (size_t)bti * S.nchunks * TB * ncols;
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int b = 2 * it + th;
      if (b < nb) {
        float v[kMaxChunks];
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c)
          v[c] = (c < S.nchunks) ? ld_dev(&P0[((size_t)c * TB + b) * ncols + col]) : 0.f;
        float t = 0.f;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) t += v[c];
        part[it] = t;
      }
    }
  }
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int b = 2 * it + th;
    if (b < nb) {
      const size_t bo = (size_t)(b0 + b);
      float sum = part[it];
      if (S.add1) sum = S.add1[bo * S.add_ld + col] + sum;
      if (S.add0) sum = S.add0[bo * S.add_ld + col] + sum;
      float* o = S.out + bo * S.out_ld + col;
      if (S.accumulate) sum = *o + sum;
      *o = sum;
      part[it] = sum;
    }
  }
  if (S.hist) {
    uint32_t* lh = reinterpret_cast<uint32_t*>(lds) + 16;
#pragma unroll
    for (int b = 0; b < TB; ++b)
      if (b < nb) hist_flush_one(part[b >> 1], (b & 1) == th, lh, S.hist + (size_t)(b0 + b) * kHistBins);
  }
}

template <int BT, bool WAIT, bool FP8, bool MFMA, bool MFMA2 = false>
__device__ __forceinline__ void axpy_task(const AxpyTask& T, int blk, float* lds) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i)
    if (i < T.nseg && blk >= T.seg[i].block0) s = i;
  const AxpySeg S = ax_seg(T, s);
  const int lb = blk - S.block0;
  if constexpr (MFMA && BT > 1 && !WAIT && !FP8) {
    if constexpr (MFMA2) {
      if (S.mfma_nt == 2) { axpy_mfma_block<2>(S, lb, T.batch, T.skew, lds); return; }
    } else {
      if (S.mfma_nt == 1) { axpy_mfma_block<1>(S, lb, T.batch, T.skew, lds); return; }
    }
  }
  if (S.wdt == W_BF16) {
    if (S.vec == 8) axpy_block<BT, 8, W_BF16, WAIT>(S, nullptr, nullptr, lb, T.batch, lds, &T);
    else axpy_block<BT, 1, W_BF16, WAIT>(S, nullptr, nullptr, lb, T.batch, lds, &T);
  } else if (FP8 && S.wdt == W_FP8) {
    // d % 16 == 0 (host check)
    if constexpr (FP8) {
      const float* const* sc = s == 0 ? T.seg_scale[0] : s == 1 ? T.seg_scale[1]
                             : s == 2 ? T.seg_scale[2] : T.seg_scale[3];
      axpy_block<BT, 16, W_FP8, WAIT>(S, sc[0], sc[1], lb, T.batch, lds, &T);
    }
  } else {
    if (S.vec == 4) axpy_block<BT, 4, W_F32, WAIT>(S, nullptr, nullptr, lb, T.batch, lds, &T);
    else axpy_block<BT, 1, W_F32, WAIT>(S, nullptr, nullptr, lb, T.batch, lds, &T);
  }
}

// --------------------------------------------------------------------------- //
// attention                                                                    //
// --------------------------------------------------------------------------- //

// Each key group (LPK lanes sharing a key row) keeps a running max m, sum l and
// p.V for its keys; groups merge in LDS (weight exp(m_g - M), 0 for a group that
// saw no key) and the splits of a (token, head) merge the same way.
// One (token b, head slot, key split) of the attention.  COHERENT_Q: q was written by
// other blocks of the same launch (read with device-coherent loads).  poison: the
// inputs are not trustworthy (a wait gave up), so the outputs are written as NaN.
// Returns true in every thread of the block that completed the slot: the one that
// stored the head's o (the last split to finish, or the only one), or split 0 of a
// slot whose head index is out of range; with part_only, every split (each stores
// only its piece).
// U: key rows in flight per key group (16 key groups of a 256-thread block at d_h = 128,
// bf16: U = 8 keeps a 128-key split in flight at once).
template <int WT, bool COHERENT_Q, int U = 4>
__device__ __forceinline__ bool attn_split(const AttnTask& T, int b, int slot, int split,
                                           float* lds, bool poison) {
  constexpr int VEC = (WT == W_BF16) ? 8 : 4;   // elements per 16-byte load
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cap = T.heads.host_count;
  const int dh = T.dh;
  // the list count, the head index (slot < capacity: readable) and q are independent
  // loads, issued together
  const int nslots = list_slots(T.heads);
  const int head = T.heads.idx ? T.heads.idx[slot] : slot;
  const int LPK = dh / VEC;          // lanes per key row
  const int KPW = 64 / LPK;          // keys per wave-load
  const int NG = kWaves * KPW;       // key groups in the block
  const int dg = lane % LPK, ks = lane / LPK;
  const int grp = wave * KPW + ks;
  const int k0 = split * T.per;
  const int k1 = min(k0 + T.per, T.n);
  const int len = max(k1 - k0, 0);

  float* gm = lds;                   // [NG <= 64] group max
  float* gl = lds + 64;              // [NG] group sum
  float* go = lds + 128;             // [NG][dh] group p.V; NG * dh = 256 * VEC <= 2048

  float qv[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const float* qp = &T.q[(size_t)b * T.q_ld + (size_t)slot * dh + dg * VEC + v];
    qv[v] = T.scale * (COHERENT_Q ? ld_dev(qp) : *qp);
    if (poison) qv[v] = __builtin_nanf("");
  }
  if (slot >= nslots) return false;
  // a head index outside [0, h) contributes nothing (W^O skips it too); its split 0
  // (every split with part_only) reports the slot complete
  if ((unsigned)head >= (unsigned)T.h) return T.part_only || split == 0;
  const size_t row0 = ((size_t)b * T.h + head) * (size_t)T.cap + k0;   // first key row
  constexpr int ESZ = (WT == W_BF16) ? 2 : 4;
  const char* Kb = static_cast<const char*>(T.K);
  const char* Vb = static_cast<const char*>(T.V);

  float m = -INFINITY, l = 0.f;
  float o[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) o[v] = 0.f;
  for (int base = 0; base < len; base += NG * U) {
    // raw 16-byte loads of U key and value rows, widened only where they are used
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NG + grp;
      if (j < len) {
        const size_t off = ((row0 + j) * (size_t)dh + (size_t)dg * VEC) * ESZ;
        kr[u] = ld_stream(reinterpret_cast<const uint4*>(Kb + off));
        vr[u] = ld_stream(reinterpret_cast<const uint4*>(Vb + off));
      } else {
        kr[u] = make_uint4(0u, 0u, 0u, 0u);
        vr[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    auto widen16 = [](uint4 x, float (&f)[VEC]) {
      if constexpr (WT == W_BF16) {
        unpack8(x, f);
      } else {
        f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
        f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
      }
    };
    float t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      widen16(kr[u], kf);
      float p = 0.f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) p = fmaf(qv[v], kf[v], p);
      t[u] = p;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      for (int off = LPK >> 1; off >= 1; off >>= 1) t[u] += __shfl_xor(t[u], off);
    float mc = m;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + u * NG + grp < len) mc = fmaxf(mc, t[u]);
    if (mc != -INFINITY) {
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - mc);
      l *= alpha;
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (base + u * NG + grp < len) {
          const float p = expf(t[u] - mc);
          l += p;
          float vf[VEC];
          widen16(vr[u], vf);
#pragma unroll
          for (int v = 0; v < VEC; ++v) o[v] = fmaf(p, vf[v], o[v]);
        }
      }
      m = mc;
    }
  }
  // per-group state to LDS, then merge the groups in order
  if (dg == 0) { gm[grp] = m; gl[grp] = l; }
#pragma unroll
  for (int v = 0; v < VEC; ++v) go[grp * dh + dg * VEC + v] = o[v];
  __syncthreads();
  float M = -INFINITY;
  for (int g = 0; g < NG; ++g) M = fmaxf(M, gm[g]);
  float L = 0.f, O = 0.f;
  if (tid < dh) {
    for (int g = 0; g < NG; ++g) {
      const float w = (gm[g] == -INFINITY) ? 0.f : expf(gm[g] - M);
      L = fmaf(w, gl[g], L);
      O = fmaf(w, go[g * dh + tid], O);
    }
  }
  // Each split stores its softmax piece (max, sum, p.V); the last split of each
  // (token, head) to finish combines them and stores o.
  const int w2 = dh + 2;
  if (T.nsplit == 1) {
    if (tid < dh) st_dev(&T.o[(size_t)b * T.o_ld + (size_t)slot * dh + tid], O / L);
    return true;
  }
  float* P = T.part + (((size_t)b * cap + slot) * T.nsplit + split) * w2;
  if (tid < dh) st_dev(&P[2 + tid], O);
  if (tid == 0) { st_dev(&P[0], M); st_dev(&P[1], L); }
  if (T.part_only) return true;
  int* flag = reinterpret_cast<int*>(lds + 128 + 2048);
  if (!arrive_last(&T.tickets[(size_t)b * cap + slot], (uint32_t)T.nsplit, flag)) return false;
  // combine the splits: (max, sum) of every split staged in LDS with one parallel load,
  // the p.V pieces fetched in batches of independent loads, summed in split order
  const float* P0 = T.part + ((size_t)b * cap + slot) * T.nsplit * w2;
  if (tid < T.nsplit) {
    gm[tid] = ld_dev(&P0[(size_t)tid * w2]);
    gl[tid] = ld_dev(&P0[(size_t)tid * w2 + 1]);
  }
  __syncthreads();
  float MM = -INFINITY;
  for (int sp = 0; sp < T.nsplit; ++sp) MM = fmaxf(MM, gm[sp]);
  if (tid < dh) {
    float LL = 0.f, OO = 0.f;
    constexpr int UB = 16;
    for (int s0 = 0; s0 < T.nsplit; s0 += UB) {
      float ov[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u)
        ov[u] = ld_dev(&P0[(size_t)min(s0 + u, T.nsplit - 1) * w2 + 2 + tid]);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        if (s0 + u < T.nsplit) {
          const float ms = gm[s0 + u];
          const float wgt = (ms == -INFINITY) ? 0.f : expf(ms - MM);
          LL = fmaf(wgt, gl[s0 + u], LL);
          OO = fmaf(wgt, ov[u], OO);
        }
      }
    }
    st_dev(&T.o[(size_t)b * T.o_ld + (size_t)slot * dh + tid], OO / LL);
  }
  return true;
}

// One attention block; with a done counter, the block that stores a head's o raises
// that head slot's counter.
template <int WT>
__device__ __forceinline__ void attn_task(const AttnTask& T, int blk, float* lds) {
  const int cap = T.heads.host_count;
  const int split = blk % T.nsplit;
  const int rest = blk / T.nsplit;
  const int slot = rest % cap;
  const bool stored = attn_split<WT, false>(T, rest / cap, slot, split, lds, false);
  if (T.done_ctr && stored) signal_done(T.done_ctr + (size_t)slot * kCtrStride);
}

// --------------------------------------------------------------------------- //
// top-k: histogram, classify, resolve                                          //
// --------------------------------------------------------------------------- //

__device__ __forceinline__ int topk_problem(const TopkTask& T, int blk, int per0, int* local) {
  if (T.np > 1 && blk >= per0) { *local = blk - per0; return 1; }
  *local = blk;
  return 0;
}

// hist: one block per (row, segment) adds the segment's top-digit histogram.
__device__ __forceinline__ void hist_block(const TopkProblem& P, int lb, float* lds) {
  const int tid = threadIdx.x;
  const int g = lb % P.nseg, b = lb / P.nseg;
  uint32_t* lh = reinterpret_cast<uint32_t*>(lds);
  const float* s = P.scores + (size_t)b * P.ld;
  for (int i = tid; i < kHistBins; i += kThreads) lh[i] = 0u;
  __syncthreads();
  const int j0 = g * kSegElems;
  const int j1 = min(j0 + kSegElems, P.N);
  for (int j = j0 + tid; j < j1; j += kThreads) atomicAdd(&lh[score_key(s[j]) >> kTopShift], 1u);
  __syncthreads();
  uint32_t* gh = P.hist + (size_t)b * kHistBins;
  for (int i = tid; i < kHistBins; i += kThreads) {
    const uint32_t c = lh[i];
    if (c) __hip_atomic_fetch_add(&gh[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(uint2* p, uint2 v) {
  const unsigned long long x = ((unsigned long long)v.y << 32) | v.x;
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), x, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 ld_dev_u64(const uint2* p) {
  const unsigned long long x = __hip_atomic_load(
      reinterpret_cast<unsigned long long*>(const_cast<uint2*>(p)), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)x, (uint32_t)(x >> 32));
}

// Ascending indices of the set bits of `nwords` words into idx; returns the count.
// `rows` words arrays at stride `nwords` are ORed first.  COHERENT: the words were
// written by other blocks of this launch (read with ld_dev); otherwise they are in
// LDS or were written by this block.
template <bool COHERENT>
__device__ __forceinline__ uint32_t compact_bits(const uint32_t* bits, int rows, int nwords,
                                                 int32_t* idx, uint32_t* scratch) {
  const int tid = threadIdx.x;
  constexpr int E = kWordsPerThread;
  uint32_t carry = 0u;
  for (int base = 0; base < nwords; base += kThreads * E) {
    uint32_t w[E];
    uint32_t n = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int word = base + tid * E + e;
      uint32_t x = 0u;
      if (word < nwords)
        for (int r = 0; r < rows; ++r)
          x |= COHERENT ? ld_dev(&bits[(size_t)r * nwords + word]) : bits[(size_t)r * nwords + word];
      w[e] = x;
      n += (uint32_t)__popc(x);
    }
    uint32_t tot;
    uint32_t pos = block_incl_scan(n, scratch, &tot) - n + carry;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      uint32_t x = w[e];
      const int word = base + tid * E + e;
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1u;
        idx[pos++] = word * 32 + bit;
      }
    }
    carry += tot;
  }
  return carry;
}

// Candidates [t0 + tid*E, t0 + tid*E + E), E = kCandPerThread, of a row's list, which is stored per
// segment (segment g holds segoff[g+1] - segoff[g] entries at src + g*kSegElems).
__device__ __forceinline__ void load_cand_tile(const uint2* src, const uint32_t* segoff, int nseg,
                                               uint32_t C, uint32_t t0,
                                               uint32_t (&key)[kCandPerThread],
                                               uint32_t (&ix)[kCandPerThread]) {
  const uint32_t c0 = t0 + threadIdx.x * kCandPerThread;
  int g = 0;
  if (c0 < C) {
    int lo = 0, hi = nseg - 1;   // last g with segoff[g] <= c0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (segoff[mid] <= c0) lo = mid; else hi = mid - 1;
    }
    g = lo;
  }
#pragma unroll
  for (int e = 0; e < kCandPerThread; ++e) {
    const uint32_t c = c0 + e;
    key[e] = 0u;
    ix[e] = 0xffffffffu;
    if (c < C) {
      while (g + 1 < nseg && segoff[g + 1] <= c) ++g;
      const uint2 kv = ld_dev_u64(&src[(size_t)g * kSegElems + (c - segoff[g])]);
      key[e] = kv.x;
      ix[e] = kv.y;
    }
  }
}

// Resolve a classified row (run by the last of its classify blocks): the `need`
// largest candidates of digit D1 (equal keys: lower index first) join the keys
// above D1, and the row is compacted (or published for the batch union).
__device__ __forceinline__ void resolve_row(const TopkProblem& P, int b, uint32_t D1, uint32_t need,
                                            float* lds) {
  const int tid = threadIdx.x;
  uint32_t* scratch = reinterpret_cast<uint32_t*>(lds);   // [8]
  uint32_t* bcast = scratch + 8;                          // [4]
  int* flag = reinterpret_cast<int*>(bcast + 4);          // [4]
  uint32_t* lh = scratch + 16;                            // [kLowBins]
  uint32_t* lw = lh + kLowBins;                           // [kResolveWords]
  uint32_t* segoff = lw + kResolveWords;                  // [kMaxSegs + 1]

  const int nwords = P.nwords;
  uint32_t* gbits = P.bits + (size_t)b * nwords;
  const bool words_in_lds = nwords <= kResolveWords;
  uint32_t* words = words_in_lds ? lw : gbits;
  if (words_in_lds)
    for (int w = tid; w < nwords; w += kThreads) lw[w] = ld_dev(&gbits[w]);
  const uint32_t* cc = reinterpret_cast<const uint32_t*>(P.ccount) + (size_t)b * P.nseg;
  uint32_t C = 0u;
  for (int g0 = 0; g0 < P.nseg; g0 += kThreads) {
    const int g = g0 + tid;
    const uint32_t n = (g < P.nseg) ? ld_dev(&cc[g]) : 0u;
    uint32_t tot;
    const uint32_t inc = block_incl_scan(n, scratch, &tot);
    if (g < P.nseg) segoff[g] = C + inc - n;
    C += tot;
  }
  if (tid == 0) segoff[P.nseg] = C;
  __syncthreads();

  if (need > 0u && C > 0u) {
    const uint2* src = P.cand + (size_t)b * P.nseg * kSegElems;
    const int ntiles = (int)((C + kCandTile - 1) / kCandTile);
    uint32_t key[kCandPerThread], ix[kCandPerThread];
    if (ntiles == 1) load_cand_tile(src, segoff, P.nseg, C, 0u, key, ix);
    // radix over the low 20 bits: [19:10] then [9:0]
    uint32_t T = D1 << kTopShift;
    uint32_t remaining = need;
    int hi = kTopShift;
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = hi - 10;
      __syncthreads();
      for (int i = tid; i < kLowBins; i += kThreads) lh[i] = 0u;
      __syncthreads();
      for (int t = 0; t < ntiles; ++t) {
        if (ntiles > 1) load_cand_tile(src, segoff, P.nseg, C, (uint32_t)t * kCandTile, key, ix);
#pragma unroll
        for (int e = 0; e < kCandPerThread; ++e)
          if (ix[e] != 0xffffffffu && (key[e] >> hi) == (T >> hi))
            atomicAdd(&lh[(key[e] >> shift) & (uint32_t)(kLowBins - 1)], 1u);
      }
      __syncthreads();
      constexpr int PT = kLowBins / kThreads;
      uint32_t hv[PT];
#pragma unroll
      for (int j = 0; j < PT; ++j) hv[j] = lh[kLowBins - 1 - tid * PT - j];
      uint32_t D, above;
      find_digit<PT>(hv, remaining, scratch, bcast, &D, &above);
      T |= D << shift;
      remaining -= above;
      hi = shift;
    }
    const uint32_t take = remaining;
    // index-ordered pass: keep key > T and the first `take` keys equal to T
    uint32_t carry_eq = 0u;
    for (int t = 0; t < ntiles; ++t) {
      if (ntiles > 1) load_cand_tile(src, segoff, P.nseg, C, (uint32_t)t * kCandTile, key, ix);
      uint32_t n_eq = 0u;
#pragma unroll
      for (int e = 0; e < kCandPerThread; ++e) n_eq += (ix[e] != 0xffffffffu && key[e] == T) ? 1u : 0u;
      uint32_t tot;
      uint32_t eq_before = block_incl_scan(n_eq, scratch, &tot) - n_eq + carry_eq;
#pragma unroll
      for (int e = 0; e < kCandPerThread; ++e) {
        if (ix[e] != 0xffffffffu) {
          bool sel = key[e] > T;
          if (key[e] == T) { sel = eq_before < take; ++eq_before; }
          if (sel) atomicOr(&words[ix[e] >> 5], 1u << (ix[e] & 31u));
        }
      }
      carry_eq += tot;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // (one row: its set is the union, compacted here without publishing the words)
  if (!P.unite || P.batch == 1) {
    const uint32_t n = words_in_lds
        ? compact_bits<false>(words, 1, nwords, P.idx + (size_t)b * P.k, scratch)
        : compact_bits<true>(words, 1, nwords, P.idx + (size_t)b * P.k, scratch);
    if (tid == 0) P.count[b] = (int32_t)n;
    return;
  }
  // batch union: publish this row's words, the last row to be resolved ORs all rows
  if (words_in_lds)
    for (int w = tid; w < nwords; w += kThreads) st_dev_u32(&gbits[w], lw[w]);
  if (!arrive_last(P.ticket, (uint32_t)P.batch, flag)) return;
  const uint32_t n = compact_bits<true>(P.bits, P.batch, nwords, P.idx, scratch);
  if (tid == 0) P.count[0] = (int32_t)n;
}

// classify: one block per (row, segment of kSegElems scores, 8 per thread).
__device__ __forceinline__ void classify_block(const TopkProblem& P, int lb, float* lds) {
  const int tid = threadIdx.x;
  const int g = lb % P.nseg, b = lb / P.nseg;
  uint32_t* scratch = reinterpret_cast<uint32_t*>(lds);   // [8]
  uint32_t* bcast = scratch + 8;                          // [4]
  int* flag = reinterpret_cast<int*>(bcast + 4);          // [4]
  const int N = P.N;
  const int k = min(max(P.k, 0), N);

  // digit D1 of the k-th key from the top, and how many keys of that digit are needed
  int D1;
  uint32_t need = 0u;
  if (k == 0) {
    D1 = kHistBins;          // nothing above, nothing equal
  } else if (k == N) {
    D1 = -1;                 // everything above
  } else {
    const uint32_t* gh = P.hist + (size_t)b * kHistBins;
    constexpr int PT = kHistBins / kThreads;
    uint32_t hv[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) hv[j] = gh[kHistBins - 1 - tid * PT - j];
    uint32_t D, above;
    find_digit<PT>(hv, (uint32_t)k, scratch, bcast, &D, &above);
    D1 = (int)D;
    need = (uint32_t)k - above;
  }

  const float* s = P.scores + (size_t)b * P.ld;
  const int j0 = g * kSegElems + tid * 8;
  uint32_t keys[8];
  uint32_t m8 = 0u, n_cand = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = j0 + e;
    keys[e] = (j < N) ? score_key(s[j]) : 0u;
    const int dig = (int)(keys[e] >> kTopShift);
    if (j < N && dig > D1) m8 |= 1u << e;
    if (j < N && dig == D1) ++n_cand;
  }
  uint32_t tot;
  uint32_t pos = block_incl_scan(n_cand, scratch, &tot) - n_cand;
  uint2* cand = P.cand + ((size_t)b * P.nseg + g) * kSegElems;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = j0 + e;
    if (j < N && (int)(keys[e] >> kTopShift) == D1) st_dev_u64(&cand[pos++], make_uint2(keys[e], (uint32_t)j));
  }
  // four threads fill one 32-bit word (8 elements each)
  uint32_t w = m8 << ((tid & 3) * 8);
  w |= __shfl_xor(w, 1);
  w |= __shfl_xor(w, 2);
  const int word = j0 >> 5;
  if ((tid & 3) == 0 && word < P.nwords) st_dev_u32(&P.bits[(size_t)b * P.nwords + word], w);
  if (tid == 0) st_dev_u32(reinterpret_cast<uint32_t*>(&P.ccount[(size_t)b * P.nseg + g]), tot);
  if (!arrive_last(&P.row_tickets[b], (uint32_t)P.nseg, flag)) return;
  resolve_row(P, b, (uint32_t)D1, need, lds);
}

__device__ __forceinline__ void topk_task(int stage, const TopkTask& T, int blk, float* lds) {
  const int per0 = T.p[0].batch * T.p[0].nseg;
  int lb;
  const int pi = topk_problem(T, blk, per0, &lb);
  const TopkProblem& P = pi == 0 ? T.p[0] : T.p[1];
  if (stage == T_HIST) hist_block(P, lb, lds);
  else classify_block(P, lb, lds);
}

// --------------------------------------------------------------------------- //
// the sparse step in one launch (see StreamTask)                               //
// --------------------------------------------------------------------------- //

// Dot item k: 8 gathered rows (2 per wave) dotted with y (in LDS), stored coherently
// for the attention (W^Q rows) or the W2 row sums (W1 rows) of this launch.
__device__ __forceinline__ void stream_dot(const StreamTask& T, int k, const float* ylds,
                                           bool poison) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool qrows = k < T.n_qi;
  const int base = (qrows ? k : k - T.n_qi) * kStreamDotRows;
  const RowList L = qrows ? T.LQ : T.LM;
  const uint16_t* W = static_cast<const uint16_t*>(qrows ? T.Wq : T.W1);
  float* out = qrows ? T.q : T.a;
  const int ex = L.expand;
  const int cap = L.host_count * ex;
  const int nslots = list_slots(L);
#pragma unroll 1
  for (int j = 0; j < kStreamRowsPerWave; ++j) {
    const int r = base + wave * kStreamRowsPerWave + j;
    const int slot = r / ex;
    if (r >= cap || slot >= nslots) continue;                   // wave-uniform
    const int item = L.idx ? L.idx[slot] : slot;
    if ((unsigned)item >= (unsigned)L.items) continue;          // no consumer reads it
    const long long row = (long long)item * ex + (r - slot * ex);
    float acc[1] = {0.f};
    rowdot_bf16<1, 24>(reinterpret_cast<const uint4*>(W + row * T.d), ylds, T.d, 1, lane, acc);
    float v = wave_sum(acc[0]);
    if (poison) v = __builtin_nanf("");
    if (lane == 0) st_dev(&out[r], v);
  }
}

// Sum item: one 256-column slice of the row sum over the W2 rows of one chunk of the
// neuron list (coefficients sigma(a)) or over the W^O rows of one head (coefficients
// o).  Stores the slice of its partial; the last item of the slice adds the partials
// in chunk order (W2 chunks, then heads) to y and stores y_out.
// Latency: the readiness poll goes out with the row-id staging, and the coefficient
// loads with the first rows' loads (coefficients first: loads complete in order, so
// waiting for them leaves the rows in flight); two round trips before the first FMA.
__device__ __forceinline__ void stream_sum(const StreamTask& T, int x, float* lds, int* sm,
                                           bool& poison) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave * 2 + (lane >> 5), hl = lane & 31;
  const int d = T.d, dh = T.dh;
  const int cap_a = T.LQ.host_count;
  const bool w2 = x < T.ncm * T.nslice;
  int slice, pidx, r0, r1, head = 0;
  const uint32_t* ready = nullptr;     // counter that must reach `target` first
  uint32_t target = 0;
  const uint16_t* W;
  if (w2) {
    const int chunk = x / T.nslice;
    slice = x - chunk * T.nslice;
    pidx = chunk;
    r0 = chunk * T.per_m;
    r1 = min(r0 + T.per_m, list_slots(T.LM));
    W = static_cast<const uint16_t*>(T.W2);
    if (r1 > r0) {
      // every dot item of the chunk (counted over its capacity) has stored its row dots
      const int rows_cap = min(T.per_m, T.LM.host_count - r0);
      ready = &T.ctr[(T.c_mdone + chunk) * kCtrStride];
      target = (uint32_t)((rows_cap + kStreamDotRows - 1) / kStreamDotRows) + T.extra;
    }
  } else {
    x -= T.ncm * T.nslice;
    const int slot = x / T.nslice;
    slice = x - slot * T.nslice;
    pidx = T.ncm + slot;
    r0 = slot * dh;
    r1 = r0;
    W = static_cast<const uint16_t*>(T.Wo);
    if (slot < list_slots(T.LQ)) {
      head = T.LQ.idx ? T.LQ.idx[slot] : slot;
      if ((unsigned)head < (unsigned)T.LQ.items) {
        r1 = r0 + dh;
        ready = &T.ctr[(T.c_oready + slot) * kCtrStride];
        target = 1u + T.extra;
      }
    }
  }
  int* lrow = reinterpret_cast<int*>(lds);                 // [kAxpyTile]
  float* lcoef = lds + kAxpyTile;                          // [kAxpyTile]
  float* red = lds + 2 * kAxpyTile;                        // [kAxGroups][kStreamSlice]
  const int col0 = slice * kStreamSlice + hl * 8;
  const bool active = col0 < d;
  float acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.f;
  bool first = true;
  for (int t0 = r0; t0 < r1; t0 += kAxpyTile) {
    const int tn = min(kAxpyTile, r1 - t0);
    __syncthreads();
    // the readiness poll (thread 0, first tile) goes out before the row ids
    uint32_t seen = 0xffffffffu;
    if (first && tid == 0 && ready)
      seen = __hip_atomic_load(const_cast<uint32_t*>(ready), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    for (int i = tid; i < tn; i += kThreads) {
      const int r = t0 + i;
      int row;
      if (w2) {
        const int item = T.LM.idx ? T.LM.idx[r] : r;
        row = (unsigned)item < (unsigned)T.LM.items ? item : -1;
      } else {
        row = head * dh + (r - r0);
      }
      lrow[i] = row;
    }
    if (first && tid == 0) {
      int gave_up = 0;
      if (ready && seen < target) {
        // not yet: poll until it is (bounded)
        uint32_t n = 0;
        while (__hip_atomic_load(const_cast<uint32_t*>(ready), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) < target) {
          if (n++ >= T.spins) { gave_up = 1; break; }
          __builtin_amdgcn_s_sleep(8);
        }
        if (gave_up) __hip_atomic_fetch_or(T.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      sm[2] = gave_up;
    }
    __syncthreads();
    if (first && sm[2]) poison = true;
    first = false;
    // coefficients (this thread's share of the tile), then the first rows of its row
    // group; the coefficients are stored once they arrive, the rows stay in flight
    float cf[(kAxpyTile + kThreads - 1) / kThreads];
#pragma unroll
    for (int j = 0; j < (kAxpyTile + kThreads - 1) / kThreads; ++j) {
      const int i = tid + j * kThreads;
      float c = 0.f;
      if (i < tn && lrow[i] >= 0)
        c = w2 ? activate(ld_dev(&T.a[t0 + i]), T.act) : ld_dev(&T.at.o[t0 + i]);
      cf[j] = poison ? __builtin_nanf("") : c;
    }
    uint4 w[kStreamU];
    int i0 = grp;
    auto load_rows = [&](int base) {
#pragma unroll
      for (int u = 0; u < kStreamU; ++u) {
        const int i = base + u * kAxGroups;
        const int row = (active && i < tn) ? lrow[i] : -1;
        w[u] = (row >= 0) ? ld_stream(reinterpret_cast<const uint4*>(W + (long long)row * d + col0))
                          : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    load_rows(i0);
#pragma unroll
    for (int j = 0; j < (kAxpyTile + kThreads - 1) / kThreads; ++j) {
      const int i = tid + j * kThreads;
      if (i < tn) lcoef[i] = cf[j];
    }
    __syncthreads();
    for (;;) {
#pragma unroll
      for (int u = 0; u < kStreamU; ++u) {
        const int i = i0 + u * kAxGroups;
        const float c = (i < tn) ? lcoef[i] : 0.f;
        float f[8];
        unpack8(w[u], f);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[v] = fmaf(c, f[v], acc[v]);
      }
      i0 += kAxGroups * kStreamU;
      if (i0 >= tn) break;
      load_rows(i0);
    }
  }
  // the row groups in order 0..7, then this item's partial slice
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 8; ++v) red[grp * kStreamSlice + hl * 8 + v] = acc[v];
  __syncthreads();
  const int col = slice * kStreamSlice + tid;
  if (col < d) {
    float part = 0.f;
#pragma unroll
    for (int g = 0; g < kAxGroups; ++g) part += red[g * kStreamSlice + tid];
    st_dev(&T.partial[(size_t)pidx * d + col], part);
  }
  const int P = T.ncm + cap_a;
  if (!arrive_last(&T.ctr[(T.c_stick + slice) * kCtrStride], (uint32_t)P, sm + 1)) return;
  if (col < d) {
    // all partials of the column requested at once (up to 48), summed in order
    constexpr int UB = 48;
    float t = 0.f;
    for (int p0 = 0; p0 < P; p0 += UB) {
      float v[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u)
        v[u] = (p0 + u < P) ? ld_dev(&T.partial[(size_t)(p0 + u) * d + col]) : 0.f;
#pragma unroll
      for (int u = 0; u < UB; ++u) t += v[u];
    }
    float o = T.y[col] + t;
    if (poison) o = __builtin_nanf("");
    T.y_out[col] = o;
  }
}

template <int KVT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void stream_kernel(StreamTask T) {
  extern __shared__ __align__(16) float lds[];
  int* sm = reinterpret_cast<int*>(reinterpret_cast<char*>(lds) + T.lds_union);
  const int tid = threadIdx.x;
  // y into LDS, for the dot items (staged again after an attention item, whose scratch
  // shares the region)
  auto stage_y = [&]() {
    const float4* src = reinterpret_cast<const float4*>(T.y);
    float4* dst = reinterpret_cast<float4*>(lds);
    for (int i = tid; i < (T.d >> 2); i += kThreads) dst[i] = src[i];
    __syncthreads();
  };
  stage_y();
  bool y_in_lds = true;
  bool poison = false;
  const int n_d = T.n_qi + T.n_mi;
  // Blocks are dealt to the XCDs round-robin (block b on XCD b % 8); queue q is served by
  // blocks b with (b / 8) % 8 == q, so every queue draws on every XCD and the queues
  // advance through the order at the same pace.  Block b's first item swaps the two low
  // octal digits of b: a bijection of each group of 64 blocks onto its 64 items in which
  // item % 8 is the block's queue.
  static_assert(kStreamQueues == 8, "queue mapping assumes 8 queues");
  const int queue = (blockIdx.x >> 3) & 7;
  uint32_t* claim = &T.ctr[queue * kCtrStride];
  int item = (blockIdx.x & ~63) | ((blockIdx.x & 7) << 3) | queue;
  while ((unsigned)item < (unsigned)T.n_items) {
    // queue position -> dot item index (W^Q dots, then W1 dots) or attention item
    const int a0 = T.n_qi + T.n_mfirst;        // first attention position
    const int dot = item < a0 ? item : (item >= a0 + T.n_a && item < n_d + T.n_a) ? item - T.n_a : -1;
    if (dot >= 0) {
      if (!y_in_lds) { stage_y(); y_in_lds = true; }
      stream_dot(T, dot, lds, poison);
      const int c = dot < T.n_qi ? T.c_qdone + dot * kStreamDotRows / T.dh
                                 : T.c_mdone + (dot - T.n_qi) * kStreamDotRows / T.per_m;
      signal_done(&T.ctr[c * kCtrStride]);
    } else if (item < a0 + T.n_a) {
      y_in_lds = false;
      const int x = item - a0;
      const int slot = x / T.at.nsplit, split = x - slot * T.at.nsplit;
      // the head's W^Q rows are dotted (dh / kStreamDotRows dot items)
      if (wait_ge(&T.ctr[(T.c_qdone + slot) * kCtrStride],
                  (uint32_t)(T.dh / kStreamDotRows) + T.extra, T.spins, T.fault, sm + 2))
        poison = true;
      if (attn_split<KVT, true, 8>(T.at, 0, slot, split, lds, poison)) {
        __builtin_amdgcn_s_waitcnt(0);      // o is stored
        __syncthreads();
        if (tid == 0)
          __hip_atomic_store(&T.ctr[(T.c_oready + slot) * kCtrStride], 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      stream_sum(T, item - n_d - T.n_a, lds, sm, poison);
    }
    // The next item of this block's queue is claimed only now: an item claimed earlier
    // would wait behind this one, however long it runs, while later items of its queue
    // went ahead (measured: 85 -> 80 us for the OPT-175B layer).  A claim past the end,
    // however large, ends the loop.
    if (tid == 0) {
      const uint32_t nxt = __hip_atomic_fetch_add(claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm[0] = T.grid + (int)min(nxt, (uint32_t)T.n_items) * kStreamQueues + queue;
    }
    __syncthreads();
    item = sm[0];
    __syncthreads();
  }
}

// A launch of `kernel` on `stream`.  With timing events, the runtime stamps them with
// the kernel's own start and end (no event packets around it, so a launch's timing slot
// measures the kernel as a kernel trace does); without, a plain launch.
template <typename K, typename A>
static void launch_k(K kernel, int grid, int lds_bytes, void* stream, void* ev0, void* ev1,
                     const A& args) {
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), (uint32_t)lds_bytes,
                          static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev0),
                          static_cast<hipEvent_t>(ev1), 0u, args);
  else
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), lds_bytes,
                       static_cast<hipStream_t>(stream), args);
}

int launch_stream(int kvdt, const StreamTask& t, int grid, int lds_bytes, void* stream,
                  void* ev0, void* ev1) {
  if (kvdt == W_BF16)
    launch_k(stream_kernel<W_BF16>, grid, lds_bytes, stream, ev0, ev1, t);
  else
    launch_k(stream_kernel<W_F32>, grid, lds_bytes, stream, ev0, ev1, t);
  return (int)hipGetLastError();
}

int stream_occupancy(int kvdt, int lds_bytes) {
  int n = 0;
  const hipError_t e = kvdt == W_BF16
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stream_kernel<W_BF16>, kThreads, lds_bytes)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stream_kernel<W_F32>, kThreads, lds_bytes);
  return e == hipSuccess ? n : 0;
}

uint32_t* fault_word() {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(dv_fault)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return static_cast<uint32_t*>(ptrs[dev]);
}

int fault_take(void* stream, uint32_t* value) {
  *value = 0u;
  uint32_t* p = fault_word();
  if (!p) return (int)hipErrorInvalidValue;
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return (int)e;
  e = hipMemcpy(value, p, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return (int)e;
  if (*value) {
    const uint32_t zero = 0u;
    e = hipMemcpy(p, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
  }
  return (int)e;
}

// --------------------------------------------------------------------------- //
// phase kernel                                                                 //
// --------------------------------------------------------------------------- //

template <int FLAGS, int BT>
__device__ __forceinline__ void phase_body(const PhaseArgs& a, float* lds) {
  const int blk = blockIdx.x;
  if constexpr ((FLAGS & T_ZERO) != 0) {
    if (blk >= a.b_zero && blk < a.b_zero + a.zero.blocks) {
      for (int i = (blk - a.b_zero) * kThreads + threadIdx.x; i < a.zero.words;
           i += a.zero.blocks * kThreads)
        a.zero.ptr[i] = 0u;
      return;
    }
  }
  if constexpr ((FLAGS & T_ROWDOT) != 0) {
    if (blk >= a.b_rowdot && blk < a.b_rowdot + a.rowdot.blocks) {
      rowdot_task<BT, (FLAGS & T_FP8) != 0, (FLAGS & T_KV) != 0>(a.rowdot, blk - a.b_rowdot, lds);
      return;
    }
  }
  if constexpr ((FLAGS & (T_HIST | T_CLASSIFY)) != 0) {
    if (blk >= a.b_topk && blk < a.b_topk + a.topk.blocks) {
      topk_task(FLAGS & (T_HIST | T_CLASSIFY), a.topk, blk - a.b_topk, lds);
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
      axpy_task<BT, (FLAGS & T_WAIT) != 0, (FLAGS & T_FP8) != 0, (FLAGS & T_MFMA) != 0,
                (FLAGS & T_MFMA2) != 0>(a.axpy, blk - a.b_axpy, lds);
      return;
    }
  }
}

// (The waiting launch over fp8 rows, whose 16-column lanes need more registers, takes
// the kernel without the 8-wave target even for one token: its grid is smaller, 24
// column slices against 48.)
// Residency is also bounded by scalar registers: measured on MI355X with 256-thread
// blocks of <= 64 VGPRs, a kernel of at most 80 SGPRs keeps 8 blocks per CU resident,
// one of 84 only 7.  The launch descriptor would otherwise take about 85, so every
// launch mix is capped at 80 except the row dots, whose vector registers hold them
// to 3 waves per SIMD anyway (they get a kernel of their own without the cap).  With
// one token per block the mixes are also held to 64 VGPRs (8 waves per SIMD); with
// 2 or 4 tokens per block they need more and get a kernel without that target.
template <int FLAGS, int BT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_sgpr(80), amdgpu_waves_per_eu(8, 8)))
void phase_kernel(PhaseArgs a) {
  extern __shared__ float lds[];
  phase_body<FLAGS, BT>(a, lds);
}

template <int FLAGS, int BT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_sgpr(80)))
void phase_kernel_bt(PhaseArgs a) {
  extern __shared__ float lds[];
  phase_body<FLAGS, BT>(a, lds);
}

template <int FLAGS, int BT>
__global__ __launch_bounds__(kThreads) void rowdot_kernel(PhaseArgs a) {
  extern __shared__ float lds[];
  phase_body<FLAGS, BT>(a, lds);
}

// The row dots with the KV stores, one token per block: held to 3 waves per SIMD like
// the plain row dots (the store path would otherwise take it past 168 registers, to 2;
// the cap costs two spilled values outside the load loop).  Larger token tiles run
// at 2 waves either way and use rowdot_kernel.
template <int FLAGS, int BT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void rowdot_kv_kernel(PhaseArgs a) {
  extern __shared__ float lds[];
  phase_body<FLAGS, BT>(a, lds);
}

// Matrix-core row dots (batch >= kMfmaMinBatch, bf16 rows): NT token tiles of 16.
template <int NT>
__global__ __launch_bounds__(kThreads) void rowdot_mfma_kernel(PhaseArgs a) {
  extern __shared__ float lds[];
  rowdot_mfma_task<NT>(a.rowdot, lds);
}

// Matrix-core row dots with y staged in LDS (batch <= 16 NT).
template <int NT>
__global__ __launch_bounds__(kThreads) void rowdot_mfma_lds_kernel(PhaseArgs a) {
  extern __shared__ float lds[];
  rdw_task<NT>(a.rowdot, lds);
}

template <int FLAGS, int BT>
static int launch_t(const PhaseArgs& a, int grid, int lds_bytes, void* stream, void* ev0,
                    void* ev1) {
  if constexpr ((FLAGS & ~T_FP8) == (T_ROWDOT | T_KV) && BT == 1)
    launch_k(rowdot_kv_kernel<FLAGS, BT>, grid, lds_bytes, stream, ev0, ev1, a);
  else if constexpr ((FLAGS & ~(T_FP8 | T_KV)) == T_ROWDOT)
    launch_k(rowdot_kernel<FLAGS, BT>, grid, lds_bytes, stream, ev0, ev1, a);
  else if constexpr (BT == 1 && (FLAGS & (T_WAIT | T_FP8)) != (T_WAIT | T_FP8))
    launch_k(phase_kernel<FLAGS, BT>, grid, lds_bytes, stream, ev0, ev1, a);
  else
    launch_k(phase_kernel_bt<FLAGS, BT>, grid, lds_bytes, stream, ev0, ev1, a);
  return (int)hipGetLastError();
}

template <int FLAGS>
static int launch_bt(int bt, const PhaseArgs& a, int grid, int lds_bytes, void* stream,
                     void* ev0, void* ev1) {
  switch (bt) {
    case 1: return launch_t<FLAGS, 1>(a, grid, lds_bytes, stream, ev0, ev1);
    case 2: return launch_t<FLAGS, 2>(a, grid, lds_bytes, stream, ev0, ev1);
    default: return launch_t<FLAGS, 4>(a, grid, lds_bytes, stream, ev0, ev1);
  }
}

int launch_phase(int flags, int bt, const PhaseArgs& a, int grid, int lds_bytes, void* stream,
                 void* ev0, void* ev1) {
  switch (flags) {
    case T_ROWDOT:
      if (a.rowdot.mfma_nt == 3 || a.rowdot.mfma_nt == 4) {
        if (a.rowdot.mfma_nt == 3)
          launch_k(rowdot_mfma_lds_kernel<1>, grid, lds_bytes, stream, ev0, ev1, a);
        else
          launch_k(rowdot_mfma_lds_kernel<2>, grid, lds_bytes, stream, ev0, ev1, a);
        return (int)hipGetLastError();
      }
      if (a.rowdot.mfma_nt > 0) {
        if (a.rowdot.mfma_nt == 1)
          launch_k(rowdot_mfma_kernel<1>, grid, lds_bytes, stream, ev0, ev1, a);
        else
          launch_k(rowdot_mfma_kernel<2>, grid, lds_bytes, stream, ev0, ev1, a);
        return (int)hipGetLastError();
      }
      return launch_bt<T_ROWDOT>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_AXPY: return launch_bt<T_AXPY>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_ATTN | T_AXPY: return launch_bt<T_ATTN | T_AXPY>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_ATTN | T_AXPY | T_WAIT: return launch_bt<T_ATTN | T_AXPY | T_WAIT>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_ATTN | T_AXPY | T_WAIT | T_FP8:
      return launch_bt<T_ATTN | T_AXPY | T_WAIT | T_FP8>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_AXPY | T_CLASSIFY: return launch_bt<T_AXPY | T_CLASSIFY>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_ROWDOT | T_FP8: return launch_bt<T_ROWDOT | T_FP8>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_ROWDOT | T_KV: return launch_bt<T_ROWDOT | T_KV>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_ROWDOT | T_KV | T_FP8:
      return launch_bt<T_ROWDOT | T_KV | T_FP8>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_AXPY | T_FP8: return launch_bt<T_AXPY | T_FP8>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    case T_AXPY | T_CLASSIFY | T_FP8:
      return launch_bt<T_AXPY | T_CLASSIFY | T_FP8>(bt, a, grid, lds_bytes, stream, ev0, ev1);
    // matrix-core row sums: batches of at least kAxMfmaMinBatch tokens (bt 4)
    case T_AXPY | T_MFMA:
      return bt == 4 ? launch_t<T_AXPY | T_MFMA, 4>(a, grid, lds_bytes, stream, ev0, ev1) : (int)hipErrorInvalidValue;
    case T_ATTN | T_AXPY | T_MFMA:
      return bt == 4 ? launch_t<T_ATTN | T_AXPY | T_MFMA, 4>(a, grid, lds_bytes, stream, ev0, ev1)
                     : (int)hipErrorInvalidValue;
    case T_AXPY | T_CLASSIFY | T_MFMA:
      return bt == 4 ? launch_t<T_AXPY | T_CLASSIFY | T_MFMA, 4>(a, grid, lds_bytes, stream, ev0, ev1)
                     : (int)hipErrorInvalidValue;
    // 32 tokens per matrix-core row-sum block (batch > 16)
    case T_AXPY | T_MFMA | T_MFMA2:
      return bt == 4 ? launch_t<T_AXPY | T_MFMA | T_MFMA2, 4>(a, grid, lds_bytes, stream, ev0, ev1)
                     : (int)hipErrorInvalidValue;
    case T_ATTN | T_AXPY | T_MFMA | T_MFMA2:
      return bt == 4 ? launch_t<T_ATTN | T_AXPY | T_MFMA | T_MFMA2, 4>(a, grid, lds_bytes, stream, ev0, ev1)
                     : (int)hipErrorInvalidValue;
    case T_AXPY | T_CLASSIFY | T_MFMA | T_MFMA2:
      return bt == 4 ? launch_t<T_AXPY | T_CLASSIFY | T_MFMA | T_MFMA2, 4>(a, grid, lds_bytes, stream, ev0, ev1)
                     : (int)hipErrorInvalidValue;
    case T_ATTN: return launch_t<T_ATTN, 1>(a, grid, lds_bytes, stream, ev0, ev1);
    case T_ZERO: return launch_t<T_ZERO, 1>(a, grid, lds_bytes, stream, ev0, ev1);
    case T_HIST: return launch_t<T_HIST, 1>(a, grid, lds_bytes, stream, ev0, ev1);
    case T_CLASSIFY: return launch_t<T_CLASSIFY, 1>(a, grid, lds_bytes, stream, ev0, ev1);
    default: return (int)hipErrorInvalidValue;
  }
}

// Blocks of the kernel that runs (flags, bt) with lds_bytes of LDS that one CU holds
// at once, as the runtime computes it from the kernel's registers and LDS.
template <int FLAGS, int BT>
static int occupancy_t(int lds_bytes) {
  int n = 0;
  hipError_t e;
  if constexpr ((FLAGS & ~T_FP8) == (T_ROWDOT | T_KV) && BT == 1)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rowdot_kv_kernel<FLAGS, BT>, kThreads,
                                                     lds_bytes);
  else if constexpr ((FLAGS & ~(T_FP8 | T_KV)) == T_ROWDOT)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rowdot_kernel<FLAGS, BT>, kThreads, lds_bytes);
  else if constexpr (BT == 1 && (FLAGS & (T_WAIT | T_FP8)) != (T_WAIT | T_FP8))
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, phase_kernel<FLAGS, BT>, kThreads, lds_bytes);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, phase_kernel_bt<FLAGS, BT>, kThreads, lds_bytes);
  return e == hipSuccess ? n : 0;
}

template <int FLAGS>
static int occupancy_bt(int bt, int lds_bytes) {
  switch (bt) {
    case 1: return occupancy_t<FLAGS, 1>(lds_bytes);
    case 2: return occupancy_t<FLAGS, 2>(lds_bytes);
    default: return occupancy_t<FLAGS, 4>(lds_bytes);
  }
}

int phase_occupancy(int flags, int bt, int lds_bytes) {
  switch (flags) {
    case T_ATTN | T_AXPY | T_WAIT: return occupancy_bt<T_ATTN | T_AXPY | T_WAIT>(bt, lds_bytes);
    case T_ATTN | T_AXPY | T_WAIT | T_FP8:
      return occupancy_bt<T_ATTN | T_AXPY | T_WAIT | T_FP8>(bt, lds_bytes);
    default: return 0;
  }
}

}  // namespace dv
