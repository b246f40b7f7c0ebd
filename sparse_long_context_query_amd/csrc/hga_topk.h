// Top-k of a wave's worth of scores by (score descending, index ascending),
// shared by the selection kernels and the decode attention kernel (gfx950,
// wave64).  The rule is the one the library implements for the history
// blocks: the k best scores, ties to the lower block index, emitted in
// ascending index order.
#pragma once

#include "hga_internal.h"

namespace hga {

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

// The k best of nb scores (nb <= 64 E) by (score desc, index asc), written
// ascending to out[0, k): one wave finds the k-th largest score thr (with
// multiplicity) by a bitwise search over the 32-bit score order held in its
// registers, then keeps every score above thr and the lowest-index ties at
// thr, compacting them in index order with ballots.  Called by the 64
// threads of one wave; `score` may be in LDS or global memory.  With
// `payload`, out receives payload[i] instead of each kept index i (its
// entries are requested together with the scores).
template <int E>
__device__ __forceinline__ void wave_topk(const float* score, int nb, int K, int32_t* out,
                                          int lane, const int32_t* payload = nullptr) {
  uint32_t v[E];
  float sv[E];
  int32_t pv[E];
  // unconditional loads (index clamped) so that all E are in flight at once
#pragma unroll
  for (int e = 0; e < E; ++e) sv[e] = score[min(64 * e + lane, nb - 1)];
  if (payload != nullptr) {
#pragma unroll
    for (int e = 0; e < E; ++e) pv[e] = payload[min(64 * e + lane, nb - 1)];
  }
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
    if (take) out[count + __popcll(m & below)] = payload != nullptr ? pv[e] : i;
    count += __popcll(m);
    ties += __popcll(meq);
  }
}

}  // namespace hga
