// Block summaries (a1), query-block means + top-k selection (a2, a3) and the
// standalone block gather (a4) of HGA, for gfx950.
//
// [JA] 深掘り分析: per-block summaries of the history stay resident on the
// GPU and grow slowly with length.  [JA] 背景と概要 / [FR] Contexte: each
// query block attends to a bounded set of history tokens that is loaded in
// a targeted way rather than by a full scan.  Summary = mean key of the
// block per KV head; score = dot product with the query block's mean query;
// ties go to the lower block index.
#include <hip/hip_runtime.h>

#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = 256;

// Where the query rows of selection unit j are and where its k indices go:
// q rows qS*(b*Hq + h) + q0 + j*qstep + [0, nrows) (q holds qS rows per
// head), output row out_units*(b*Hkv + g) + out_j0 + j of sel, nb candidate
// blocks.  A segment's unit is a query block; a decode step's single unit is
// its new tokens.
struct SelGeom {
  int qS, q0, qstep, nrows;
  int out_units, out_j0;
  int nb;
  // several segments in one launch (per_seg > 0): unit u is query block
  // u % per_seg of segment seg0 + u / per_seg, whose rows start at
  // seg * seg_len and whose candidates are its seg * seg_len / bh closed
  // blocks; q0, out_j0 and nb above are then per unit, nb giving the most
  // candidates of any unit
  int per_seg, seg0, seg_len, bh;
};

// ---------------------------------------------------------------------------
// a1: summ[b,g,i,:] = mean of the Bh keys of block i.
// One block of threads per (history block, KV head, sequence).  Threads read
// rows in 16-byte pieces: C pieces per row, R rows in flight per pass; the
// R partial sums are then folded through LDS.  HBM-bound.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void summarize_kernel(
    const T* __restrict__ k, float* __restrict__ summ, int S, int Bh, int Hkv,
    int nblk, int blk_begin, int row_shift) {
  constexpr int E = Vec16<T>::N;
  constexpr int C = D / E;
  constexpr int R = kThreads / C;
  __shared__ float part[R][D + 1];

  const int i = blk_begin + blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  // rows per (b, g): S; block i's first row: i * Bh + row_shift
  const T* base = k + ((size_t)(b * Hkv + g) * S + (size_t)(i * Bh + row_shift)) * D;
  const int c = threadIdx.x % C, r = threadIdx.x / C;

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int row = r; row < Bh; row += R) {
    float f[E];
    Vec16<T>::load(base + (size_t)row * D + c * E, f);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += f[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) part[r][c * E + e] = acc[e];
  __syncthreads();
  const float inv = 1.0f / (float)Bh;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float s = 0.f;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) s += part[rr][d];
    summ[((size_t)(b * Hkv + g) * nblk + i) * D + d] = s * inv;
  }
}

// Orderable 64-bit key: high word = score mapped to an unsigned order
// (larger score -> larger word), low word = ~index so that equal scores
// rank the lower index higher.  Sorting keys descending yields the
// (score desc, index asc) ranking.
__device__ __forceinline__ unsigned long long rank_key(float s, int idx) {
  s = s + 0.0f;  // -0 -> +0 so that zero scores tie exactly
  uint32_t u = __float_as_uint(s);
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (uint32_t)(0xffffffffu - (uint32_t)idx);
}

// In-LDS bitonic sort of n (power of two) 64-bit keys, descending.
__device__ void bitonic_desc(unsigned long long* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kThreads) {
        int ixj = i ^ j;
        if (ixj > i) {
          unsigned long long x = a[i], y = a[ixj];
          bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) { a[i] = y; a[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
}

// Orderable 32-bit image of a score (larger score -> larger word; -0 and +0
// tie); 0 lies below every finite score.
__device__ __forceinline__ uint32_t score_ord(float s) {
  s = s + 0.0f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The k-th largest of the 64*E words held by one wave, counted with
// multiplicity (E per lane, unused slots 0): the largest T with
// #{words >= T} >= k, found bit by bit from the top.
template <int E>
__device__ __forceinline__ uint32_t wave_kth_largest32(const uint32_t (&v)[E], int k) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c += __popcll(__ballot(v[e] >= cand));
    if (c >= k) t = cand;
  }
  return t;
}

// qbar[d] = mean over the G heads of group g and the nrows query rows of
// unit j of q (float32): every row load of a thread in flight at once, then
// an LDS fold over the R row slots.  Ends with a barrier (qbar is ready).
template <typename T, int D>
__device__ __forceinline__ void group_query_mean(const T* __restrict__ q, const SelGeom& geo,
                                                 int b, int g, int j, int Hq, int G,
                                                 float (*part)[D + 1], float* qbar) {
  constexpr int EL = Vec16<T>::N;
  constexpr int C = D / EL;
  constexpr int R = kThreads / C;
  const int c = threadIdx.x % C, r = threadIdx.x / C;
  float acc[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) acc[e] = 0.f;
  const int rows = G * geo.nrows;
  constexpr int U = 16;  // row loads in flight per thread (raw 16-byte vectors)
  for (int row0 = r; row0 < rows; row0 += U * R) {
    uint4 f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = row0 + u * R;
      if (row < rows) {
        const int hh = row / geo.nrows, tt = row % geo.nrows;
        f[u] = *reinterpret_cast<const uint4*>(
            q + ((size_t)(b * Hq + g * G + hh) * geo.qS + geo.q0 + j * geo.qstep + tt) * D +
            c * EL);
      } else {
        f[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[EL];
      Vec16<T>::load(reinterpret_cast<const T*>(&f[u]), x);
#pragma unroll
      for (int e = 0; e < EL; ++e) acc[e] += x[e];
    }
  }
#pragma unroll
  for (int e = 0; e < EL; ++e) part[r][c * EL + e] = acc[e];
  __syncthreads();
  const float inv = 1.0f / (float)rows;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float sum = 0.f;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) sum += part[rr][d];
    qbar[d] = sum * inv;
  }
  __syncthreads();
}

// The k best of nb scores (nb <= 64 E) by (score desc, index asc), written
// ascending to out[0, k): one wave finds the k-th largest score thr (with
// multiplicity) by a bitwise search over the 32-bit score order held in its
// registers, then keeps every score above thr and the lowest-index ties at
// thr, compacting them in index order with ballots.  Called by the 64
// threads of one wave; `score` may be in LDS or global memory.
template <int E>
__device__ __forceinline__ void wave_topk(const float* score, int nb, int K, int32_t* out,
                                          int lane) {
  uint32_t v[E];
  float sv[E];
  // unconditional loads (index clamped) so that all E are in flight at once
#pragma unroll
  for (int e = 0; e < E; ++e) sv[e] = score[min(64 * e + lane, nb - 1)];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = 64 * e + lane < nb ? score_ord(sv[e]) : 0u;
  const uint32_t thr = wave_kth_largest32<E>(v, K);
  int gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) gt += __popcll(__ballot(v[e] > thr));
  const int need = K - gt;
  const unsigned long long below = (1ull << lane) - 1ull;
  int count = 0, ties = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = 64 * e + lane;
    const bool ok = i < nb;
    const bool eq = ok && v[e] == thr;
    const unsigned long long meq = __ballot(eq);
    const bool take = (ok && v[e] > thr) || (eq && ties + __popcll(meq & below) < need);
    const unsigned long long m = __ballot(take);
    if (take) out[count + __popcll(m & below)] = i;
    count += __popcll(m);
    ties += __popcll(meq);
  }
}

// ---------------------------------------------------------------------------
// a2 + a3: one block of threads per (unit j, KV head g, sequence b); a unit
// is a query block of a segment, or the new tokens of a decode step.
//   1. qbar = mean of q over the G heads of the group and the unit's rows
//      (float32; every row load of a thread in flight at once, then an LDS
//      fold); the summary row of each thread's first candidate
//      is requested before the q rows so that both round trips overlap;
//   2. score_i = qbar . summ_i (unscaled), one candidate per thread, qbar
//      broadcast from LDS;
//   3. for up to 1024 candidates one wave finds the k-th largest score T
//      (with multiplicity) by a bitwise search over the 32-bit score order
//      held in its registers; beyond that the score and index form one
//      orderable 64-bit key and an LDS bitonic sort over all threads gives
//      the k-th largest key;
//   4. the k best by (score desc, index asc) -- every score above T plus the
//      lowest-index ties at T, or every key >= the k-th key -- are compacted
//      in index order (ballots), so the output is ascending; padded with -1.
// E = keys per lane of the register search (0 selects the LDS sort).
// ---------------------------------------------------------------------------
template <typename T, int D, int E>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const T* __restrict__ q, const float* __restrict__ summ,
    int32_t* __restrict__ sel, SelGeom geo, int K, int Hq, int Hkv, int G, int nblk) {
  constexpr int EL = Vec16<T>::N;
  constexpr int C = D / EL;
  constexpr int R = kThreads / C;
  extern __shared__ unsigned long long keys[];  // LDS sort only
  __shared__ float part[R][D + 1];
  __shared__ __attribute__((aligned(16))) float qbar[D];
  __shared__ float s_score[kMaxCandidates];
  __shared__ unsigned long long s_thresh;

  int j = blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  if (geo.per_seg > 0) {
    const int seg = geo.seg0 + j / geo.per_seg;
    j %= geo.per_seg;
    geo.q0 = seg * geo.seg_len;
    geo.out_j0 = seg * geo.per_seg;
    geo.nb = geo.q0 / geo.bh;
  }
  const int nb = geo.nb;
  int32_t* out = sel + ((size_t)(b * Hkv + g) * geo.out_units + geo.out_j0 + j) * K;

  if (nb <= K) {  // every history block is taken (none at seg 0)
    for (int t = threadIdx.x; t < K; t += kThreads) out[t] = (t < nb) ? t : -1;
    return;
  }

  // 2a. the first candidate's summary row of every thread, requested first
  constexpr int NV = D / 4;
  const float* sbase = summ + (size_t)(b * Hkv + g) * nblk * D;
  float4 srow0[NV];
  {
    const int i = threadIdx.x < nb ? threadIdx.x : 0;
    const float4* rowp = reinterpret_cast<const float4*>(sbase + (size_t)i * D);
#pragma unroll
    for (int u = 0; u < NV; ++u) srow0[u] = rowp[u];
  }

  // 1. query-block mean over (head in group, token in block)
  group_query_mean<T, D>(q, geo, b, g, j, Hq, G, part, qbar);

  // 2. scores, one candidate per thread
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    float sc = 0.f;
    if (i == threadIdx.x) {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const float4 qv = *reinterpret_cast<const float4*>(&qbar[4 * u]);
        sc += qv.x * srow0[u].x + qv.y * srow0[u].y + qv.z * srow0[u].z + qv.w * srow0[u].w;
      }
    } else {
      const float4* rowp = reinterpret_cast<const float4*>(sbase + (size_t)i * D);
      constexpr int UV = 16;
#pragma unroll
      for (int v0 = 0; v0 < NV; v0 += UV) {
        float4 x[UV];
#pragma unroll
        for (int u = 0; u < UV; ++u) x[u] = rowp[v0 + u];
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          const float4 qv = *reinterpret_cast<const float4*>(&qbar[4 * (v0 + u)]);
          sc += qv.x * x[u].x + qv.y * x[u].y + qv.z * x[u].z + qv.w * x[u].w;
        }
      }
    }
    s_score[i] = sc;
  }
  __syncthreads();

  if constexpr (E > 0) {
    // 3. + 4. the k-th largest score and the k best, one wave
    if (threadIdx.x < 64) wave_topk<E>(s_score, nb, K, out, threadIdx.x);
  } else {
    // 3. the k-th largest (score, index) key by an LDS sort
    int W = 1;
    while (W < nb) W <<= 1;
    for (int i = threadIdx.x; i < W; i += kThreads)
      keys[i] = i < nb ? rank_key(s_score[i], i) : 0ull;
    __syncthreads();
    bitonic_desc(keys, W);
    if (threadIdx.x == 0) s_thresh = keys[K - 1];
    __syncthreads();
    // 4. the k best in index order
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const unsigned long long thr = s_thresh;
      int count = 0;
      for (int base = 0; base < nb; base += 64) {
        const int i = base + lane;
        const bool take = i < nb && rank_key(s_score[i], i) >= thr;
        const unsigned long long m = __ballot(take);
        const int pos = count + __popcll(m & ((1ull << lane) - 1ull));
        if (take && pos < K) out[pos] = i;  // keys are unique: exactly K are taken
        count += __popcll(m);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Selection of a decode step, which has a single unit per (b, g) but up to
// 1,024 candidates: two launches so that reading the summaries spreads over
// many CUs.  score_kernel: one candidate per thread, 256 per block of
// threads, writes the fp32 scores (the same dot products select_kernel
// forms); topk_kernel: one wave per (b, g) picks the k best (wave_topk).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void score_kernel(
    const T* __restrict__ q, const float* __restrict__ summ, float* __restrict__ scores,
    SelGeom geo, int Hq, int Hkv, int G, int nblk) {
  constexpr int EL = Vec16<T>::N;
  constexpr int C = D / EL;
  constexpr int R = kThreads / C;
  constexpr int NV = D / 4;
  __shared__ float part[R][D + 1];
  __shared__ __attribute__((aligned(16))) float qbar[D];
  const int g = blockIdx.y, b = blockIdx.z;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  // the candidate's summary row first, so that it overlaps the query mean
  const float4* rowp = reinterpret_cast<const float4*>(
      summ + ((size_t)(b * Hkv + g) * nblk + (i < geo.nb ? i : 0)) * D);
  float4 x[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) x[u] = rowp[u];
  group_query_mean<T, D>(q, geo, b, g, 0, Hq, G, part, qbar);
  float sc = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const float4 qv = *reinterpret_cast<const float4*>(&qbar[4 * u]);
    sc += qv.x * x[u].x + qv.y * x[u].y + qv.z * x[u].z + qv.w * x[u].w;
  }
  if (i < geo.nb) scores[(size_t)(b * Hkv + g) * nblk + i] = sc;
}

template <int E>
__global__ __launch_bounds__(64) void topk_kernel(const float* __restrict__ scores,
                                                  int32_t* __restrict__ sel, int nb, int K,
                                                  int Hkv, int nblk) {
  const int g = blockIdx.y, b = blockIdx.z;
  wave_topk<E>(scores + (size_t)(b * Hkv + g) * nblk, nb, K, sel + (size_t)(b * Hkv + g) * K,
               threadIdx.x);
}

// ---------------------------------------------------------------------------
// a4 standalone: copy the chosen Bh x D slabs of K and V, one block of
// threads per (slot, query block, KV head, sequence), 16-byte vectors.
// Entries outside [0, nb) are treated as padding and give zeros.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v,
    const int32_t* __restrict__ sel, uint4* __restrict__ ko,
    uint4* __restrict__ vo, int S, int Bh, int K, int Hkv, int nqb,
    int nqb_all, int seg, int row16, int nb) {
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int t = w % K;
  const int j = (w / K) % nqb;
  const int g = (w / (K * nqb)) % Hkv;
  const int b = w / (K * nqb * Hkv);
  const int blk = sel[((size_t)(b * Hkv + g) * nqb_all + (size_t)seg * nqb + j) * K + t];
  const size_t n16 = (size_t)Bh * row16;
  const size_t dst = (size_t)w * n16;
  if (blk < 0 || blk >= nb) {
    const uint4 z = make_uint4(0, 0, 0, 0);
    for (size_t i = threadIdx.x; i < n16; i += kThreads) { ko[dst + i] = z; vo[dst + i] = z; }
    return;
  }
  const size_t src = ((size_t)(b * Hkv + g) * S + (size_t)blk * Bh) * row16;
  size_t i = threadIdx.x;
  for (; i + 3 * kThreads < n16; i += 4 * kThreads) {
    uint4 a0 = k[src + i], a1 = k[src + i + kThreads], a2 = k[src + i + 2 * kThreads],
          a3 = k[src + i + 3 * kThreads];
    uint4 c0 = v[src + i], c1 = v[src + i + kThreads], c2 = v[src + i + 2 * kThreads],
          c3 = v[src + i + 3 * kThreads];
    ko[dst + i] = a0; ko[dst + i + kThreads] = a1; ko[dst + i + 2 * kThreads] = a2;
    ko[dst + i + 3 * kThreads] = a3;
    vo[dst + i] = c0; vo[dst + i + kThreads] = c1; vo[dst + i + 2 * kThreads] = c2;
    vo[dst + i + 3 * kThreads] = c3;
  }
  for (; i < n16; i += kThreads) { ko[dst + i] = k[src + i]; vo[dst + i] = v[src + i]; }
}

template <typename T, int D>
hipError_t summarize_t(const Prob& p, const void* k, int b0, int b1, float* summ,
                       hipStream_t st, int row_shift) {
  dim3 grid(b1 - b0, p.Hkv, p.B);
  HGA_LAUNCH(HGA_K_SUMMARIZE, (summarize_kernel<T, D>), grid, dim3(kThreads), 0, st,
                     (const T*)k, summ, p.kv_rows, p.Bh, p.Hkv, p.nblk, b0, row_shift);
  return hipGetLastError();
}

template <typename T, int D, int E>
hipError_t select_launch(const Prob& p, const void* q, const float* summ, const SelGeom& geo,
                         int units, int32_t* sel, size_t shm, hipStream_t st) {
  if (shm > 32768) {  // large candidate sets need more than the default LDS cap
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel<T, D, E>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(kMaxCandidates * sizeof(unsigned long long)));
    if (e != hipSuccess) return e;
  }
  dim3 grid(units, p.Hkv, p.B);
  HGA_LAUNCH(HGA_K_SELECT, (select_kernel<T, D, E>), grid, dim3(kThreads), shm, st,
             (const T*)q, summ,
                     sel, geo, p.K, p.Hq, p.Hkv, p.G, p.nblk);
  return hipGetLastError();
}

// Register search for up to 1024 candidates (E = 1..16 keys per lane), LDS
// sort beyond.
template <typename T, int D>
hipError_t select_t(const Prob& p, const void* q, const float* summ, const SelGeom& geo,
                    int units, int32_t* sel, hipStream_t st) {
  const int nb = geo.nb;
  int W = 64;
  while (W < nb) W <<= 1;
  if (nb <= p.K || W <= 64) return select_launch<T, D, 1>(p, q, summ, geo, units, sel, 0, st);
  if (W <= 128) return select_launch<T, D, 2>(p, q, summ, geo, units, sel, 0, st);
  if (W <= 256) return select_launch<T, D, 4>(p, q, summ, geo, units, sel, 0, st);
  if (W <= 512) return select_launch<T, D, 8>(p, q, summ, geo, units, sel, 0, st);
  if (W <= 1024) return select_launch<T, D, 16>(p, q, summ, geo, units, sel, 0, st);
  return select_launch<T, D, 0>(p, q, summ, geo, units, sel,
                                (size_t)W * sizeof(unsigned long long), st);
}

hipError_t select_any(const Prob& p, const void* q, const float* summ, const SelGeom& geo,
                      int units, int32_t* sel, hipStream_t st) {
  if (p.dtype == HGA_BF16)
    return p.D == 64 ? select_t<__bf16, 64>(p, q, summ, geo, units, sel, st)
                     : select_t<__bf16, 128>(p, q, summ, geo, units, sel, st);
  return p.D == 64 ? select_t<float, 64>(p, q, summ, geo, units, sel, st)
                   : select_t<float, 128>(p, q, summ, geo, units, sel, st);
}

}  // namespace

hipError_t launch_summarize(const Prob& p, const void* k, int b0, int b1, float* summ,
                            hipStream_t st, int row_shift) {
  if (b1 <= b0) return hipSuccess;
  if (p.dtype == HGA_BF16)
    return p.D == 64 ? summarize_t<__bf16, 64>(p, k, b0, b1, summ, st, row_shift)
                     : summarize_t<__bf16, 128>(p, k, b0, b1, summ, st, row_shift);
  return p.D == 64 ? summarize_t<float, 64>(p, k, b0, b1, summ, st, row_shift)
                   : summarize_t<float, 128>(p, k, b0, b1, summ, st, row_shift);
}

hipError_t launch_select(const Prob& p, const void* q, const float* summ, int seg,
                         int32_t* sel, hipStream_t st) {
  // unit j = query block j of the segment, rows [t0 + j Bq, t0 + (j+1) Bq)
  const int t0 = seg * p.L;
  const SelGeom geo{p.S, t0, p.Bq, p.Bq, p.nqb_all, seg * p.nqb, t0 / p.Bh, 0, 0, 0, 0};
  return select_any(p, q, summ, geo, p.nqb, sel, st);
}

hipError_t launch_select_pass(const Prob& p, const void* q, const float* summ, int seg0,
                              int nseg, int32_t* sel, hipStream_t st) {
  // units: query block j of segment seg0 + s is unit s * nqb + j; the search
  // is sized for the last segment, which has the most candidates
  const int last = seg0 + nseg - 1;
  const SelGeom geo{p.S, 0, p.Bq, p.Bq, p.nqb_all, 0, last * p.L / p.Bh, p.nqb, seg0, p.L, p.Bh};
  return select_any(p, q, summ, geo, p.nqb * nseg, sel, st);
}

hipError_t launch_select_decode(const Prob& p, const void* q_new, int n, int t0,
                                const float* summ, int32_t* sel, float* scores,
                                hipStream_t st) {
  // one unit: the n new tokens of q_new [B, Hq, n, D]; sel is [B, Hkv, k]
  const SelGeom geo{n, 0, 0, n, 1, 0, t0 / p.Bh, 0, 0, 0, 0};
  const int nb = geo.nb;
  if (nb <= p.K || nb > 1024) return select_any(p, q_new, summ, geo, 1, sel, st);
  const dim3 grid((nb + kThreads - 1) / kThreads, p.Hkv, p.B);
  if (p.dtype == HGA_BF16) {
    if (p.D == 64)
      HGA_LAUNCH(HGA_K_SELECT, (score_kernel<__bf16, 64>), grid, dim3(kThreads), 0, st,
                         (const __bf16*)q_new, summ, scores, geo, p.Hq, p.Hkv, p.G, p.nblk);
    else
      HGA_LAUNCH(HGA_K_SELECT, (score_kernel<__bf16, 128>), grid, dim3(kThreads), 0, st,
                         (const __bf16*)q_new, summ, scores, geo, p.Hq, p.Hkv, p.G, p.nblk);
  } else {
    if (p.D == 64)
      HGA_LAUNCH(HGA_K_SELECT, (score_kernel<float, 64>), grid, dim3(kThreads), 0, st,
                         (const float*)q_new, summ, scores, geo, p.Hq, p.Hkv, p.G, p.nblk);
    else
      HGA_LAUNCH(HGA_K_SELECT, (score_kernel<float, 128>), grid, dim3(kThreads), 0, st,
                         (const float*)q_new, summ, scores, geo, p.Hq, p.Hkv, p.G, p.nblk);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g1(1, p.Hkv, p.B);
  if (nb <= 64)
    HGA_LAUNCH(HGA_K_SELECT, topk_kernel<1>, g1, dim3(64), 0, st,
               scores, sel, nb, p.K, p.Hkv, p.nblk);
  else if (nb <= 128)
    HGA_LAUNCH(HGA_K_SELECT, topk_kernel<2>, g1, dim3(64), 0, st,
               scores, sel, nb, p.K, p.Hkv, p.nblk);
  else if (nb <= 256)
    HGA_LAUNCH(HGA_K_SELECT, topk_kernel<4>, g1, dim3(64), 0, st,
               scores, sel, nb, p.K, p.Hkv, p.nblk);
  else if (nb <= 512)
    HGA_LAUNCH(HGA_K_SELECT, topk_kernel<8>, g1, dim3(64), 0, st,
               scores, sel, nb, p.K, p.Hkv, p.nblk);
  else
    HGA_LAUNCH(HGA_K_SELECT, topk_kernel<16>, g1, dim3(64), 0, st, scores, sel, nb, p.K, p.Hkv,
                       p.nblk);
  return hipGetLastError();
}

hipError_t launch_gather(const Prob& p, const void* k, const void* v, const int32_t* sel,
                         int seg, void* ko, void* vo, hipStream_t st) {
  const int esz = p.dtype == HGA_BF16 ? 2 : 4;
  const int row16 = p.D * esz / 16;
  const int nblocks = p.B * p.Hkv * p.nqb * p.K;
  const int nb = seg * p.L / p.Bh;
  HGA_LAUNCH(HGA_K_GATHER, gather_kernel, dim3(nblocks), dim3(kThreads), 0, st, (const uint4*)k,
                     (const uint4*)v, sel, (uint4*)ko, (uint4*)vo, p.S, p.Bh, p.K, p.Hkv,
                     p.nqb, p.nqb_all, seg, row16, nb);
  return hipGetLastError();
}

}  // namespace hga
