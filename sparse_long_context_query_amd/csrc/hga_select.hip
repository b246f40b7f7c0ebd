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

// ---------------------------------------------------------------------------
// a1: summ[b,g,i,:] = mean of the Bh keys of block i.
// One block of threads per (history block, KV head, sequence).  Threads read
// rows in 16-byte pieces: C pieces per row, R rows in flight per pass; the
// R partial sums are then folded through LDS.  HBM-bound.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void summarize_kernel(
    const T* __restrict__ k, float* __restrict__ summ, int S, int Bh, int Hkv,
    int nblk, int blk_begin) {
  constexpr int E = Vec16<T>::N;
  constexpr int C = D / E;
  constexpr int R = kThreads / C;
  __shared__ float part[R][D + 1];

  const int i = blk_begin + blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const T* base = k + ((size_t)(b * Hkv + g) * S + (size_t)i * Bh) * D;
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

// In-LDS bitonic sort of n (power of two) ints, ascending.
__device__ void bitonic_asc(int* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kThreads) {
        int ixj = i ^ j;
        if (ixj > i) {
          int x = a[i], y = a[ixj];
          bool asc = (i & k) == 0;
          if (asc ? (x > y) : (x < y)) { a[i] = y; a[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// a2 + a3: one block of threads per (query block j, KV head g, sequence b).
//   1. qbar = mean of q over the G heads of the group and the Bq tokens of
//      the block (float32, LDS fold as in summarize_kernel);
//   2. scores against the nb resident summaries: 16 lanes per candidate,
//      each holding D/16 dims, folded with a 16-lane shuffle reduction;
//   3. bitonic sort of the orderable keys in LDS, keep the first k;
//   4. bitonic sort of those k indices ascending, pad with -1, store.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const T* __restrict__ q, const float* __restrict__ summ,
    int32_t* __restrict__ sel, int S, int L, int Bq, int Bh, int K, int Hq,
    int Hkv, int G, int nqb_all, int nblk, int seg) {
  constexpr int E = Vec16<T>::N;
  constexpr int C = D / E;
  constexpr int R = kThreads / C;
  constexpr int DL = D / 16;
  extern __shared__ unsigned long long keys[];
  __shared__ float part[R][D + 1];
  __shared__ float qbar[D];
  __shared__ int top[kMaxTopK];

  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t0 = seg * L;
  const int nb = t0 / Bh;
  const int nqb = L / Bq;
  int32_t* out = sel + ((size_t)(b * Hkv + g) * nqb_all + (size_t)seg * nqb + j) * K;

  if (nb <= K) {  // every history block is taken (none at seg 0)
    for (int t = threadIdx.x; t < K; t += kThreads) out[t] = (t < nb) ? t : -1;
    return;
  }

  // 1. query-block mean over (head in group, token in block)
  {
    const int c = threadIdx.x % C, r = threadIdx.x / C;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    const int rows = G * Bq;
    for (int row = r; row < rows; row += R) {
      const int hh = row / Bq, tt = row % Bq;
      const T* p = q + ((size_t)(b * Hq + g * G + hh) * S + t0 + j * Bq + tt) * D + c * E;
      float f[E];
      Vec16<T>::load(p, f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += f[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) part[r][c * E + e] = acc[e];
    __syncthreads();
    const float inv = 1.0f / (float)rows;
    for (int d = threadIdx.x; d < D; d += kThreads) {
      float s = 0.f;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) s += part[rr][d];
      qbar[d] = s * inv;
    }
    __syncthreads();
  }

  // 2. scores (unscaled dot products) -> orderable keys
  int W = 1;
  while (W < nb) W <<= 1;
  {
    const int grp = threadIdx.x / 16, ln = threadIdx.x % 16;
    float qv[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) qv[e] = qbar[ln * DL + e];
    const float* srow = summ + (size_t)(b * Hkv + g) * nblk * D + ln * DL;
    for (int i = grp; i < W; i += kThreads / 16) {
      float s = 0.f;
      if (i < nb) {
        const float* p = srow + (size_t)i * D;
#pragma unroll
        for (int e = 0; e < DL; e += 4) {
          float4 x = *reinterpret_cast<const float4*>(p + e);
          s += qv[e] * x.x + qv[e + 1] * x.y + qv[e + 2] * x.z + qv[e + 3] * x.w;
        }
      }
      s += __shfl_xor(s, 8, 16);
      s += __shfl_xor(s, 4, 16);
      s += __shfl_xor(s, 2, 16);
      s += __shfl_xor(s, 1, 16);
      if (ln == 0) keys[i] = (i < nb) ? rank_key(s, i) : 0ull;
    }
  }
  __syncthreads();

  // 3. rank all candidates
  bitonic_desc(keys, W);

  // 4. the k best, ascending by index
  int KP = 1;
  while (KP < K) KP <<= 1;
  for (int t = threadIdx.x; t < KP; t += kThreads)
    top[t] = (t < K) ? (int)(0xffffffffu - (uint32_t)(keys[t] & 0xffffffffull)) : 0x7fffffff;
  __syncthreads();
  bitonic_asc(top, KP);
  for (int t = threadIdx.x; t < K; t += kThreads) out[t] = top[t];
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
                       hipStream_t st) {
  dim3 grid(b1 - b0, p.Hkv, p.B);
  ProfScope ps(HGA_K_SUMMARIZE, st);
  hipLaunchKernelGGL((summarize_kernel<T, D>), grid, dim3(kThreads), 0, st,
                     (const T*)k, summ, p.S, p.Bh, p.Hkv, p.nblk, b0);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t select_t(const Prob& p, const void* q, const float* summ, int seg,
                    int32_t* sel, hipStream_t st) {
  const int nb = seg * p.L / p.Bh;
  int W = 1;
  while (W < nb) W <<= 1;
  size_t shm = (nb > p.K) ? (size_t)W * sizeof(unsigned long long) : 0;
  if (shm > 32768) {  // large candidate sets need more than the default LDS cap
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel<T, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(kMaxCandidates * sizeof(unsigned long long)));
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.nqb, p.Hkv, p.B);
  ProfScope ps(HGA_K_SELECT, st);
  hipLaunchKernelGGL((select_kernel<T, D>), grid, dim3(kThreads), shm, st, (const T*)q,
                     summ, sel, p.S, p.L, p.Bq, p.Bh, p.K, p.Hq, p.Hkv, p.G, p.nqb_all,
                     p.nblk, seg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_summarize(const Prob& p, const void* k, int b0, int b1, float* summ,
                            hipStream_t st) {
  if (b1 <= b0) return hipSuccess;
  if (p.dtype == HGA_BF16)
    return p.D == 64 ? summarize_t<__bf16, 64>(p, k, b0, b1, summ, st)
                     : summarize_t<__bf16, 128>(p, k, b0, b1, summ, st);
  return p.D == 64 ? summarize_t<float, 64>(p, k, b0, b1, summ, st)
                   : summarize_t<float, 128>(p, k, b0, b1, summ, st);
}

hipError_t launch_select(const Prob& p, const void* q, const float* summ, int seg,
                         int32_t* sel, hipStream_t st) {
  if (p.dtype == HGA_BF16)
    return p.D == 64 ? select_t<__bf16, 64>(p, q, summ, seg, sel, st)
                     : select_t<__bf16, 128>(p, q, summ, seg, sel, st);
  return p.D == 64 ? select_t<float, 64>(p, q, summ, seg, sel, st)
                   : select_t<float, 128>(p, q, summ, seg, sel, st);
}

hipError_t launch_gather(const Prob& p, const void* k, const void* v, const int32_t* sel,
                         int seg, void* ko, void* vo, hipStream_t st) {
  const int esz = p.dtype == HGA_BF16 ? 2 : 4;
  const int row16 = p.D * esz / 16;
  const int nblocks = p.B * p.Hkv * p.nqb * p.K;
  const int nb = seg * p.L / p.Bh;
  ProfScope ps(HGA_K_GATHER, st);
  hipLaunchKernelGGL(gather_kernel, dim3(nblocks), dim3(kThreads), 0, st, (const uint4*)k,
                     (const uint4*)v, sel, (uint4*)ko, (uint4*)vo, p.S, p.Bh, p.K, p.Hkv,
                     p.nqb, p.nqb_all, seg, row16, nb);
  return hipGetLastError();
}

}  // namespace hga
