// Internal declarations of the HGA HIP library (gfx950 only).
//
// Page keys used in citations across the sources:
//   [JA] 「低VRAM長文脈ファインチューニング：階層的グローバル注意と分割バック
//        プロpagationの実践」, sns.style (Japanese edition)
//   [FR] « Ajustement fin long-contexte à faible VRAM : une approche
//        d'optimisation avec attention globale hiérarchique », sns.style
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hga.h"

namespace hga {

// Validated problem description (all derived sizes precomputed on the host).
struct Prob {
  int B, S, L, Bh, Bq, K, Hq, Hkv, D, G;
  int dtype;      // HGA_F32 / HGA_BF16
  float scale;    // softmax scale (natural-log units)
  int nqb;        // query blocks per segment  = L / Bq
  int nqb_all;    // query blocks per sequence = S / Bq
  int nblk;       // history blocks per sequence = S / Bh
  // K/V storage the step kernels read (bf16 only): rows per (b, g) and the
  // row of the segment's first key.  Full-sequence storage: kv_rows = S and
  // kv_local = -1 (a key's row is its token index).  The host tier's window
  // holds the chosen history blocks at rows slot * Bh and the segment's own
  // keys from row kv_local on.
  int kv_rows;
  int kv_local;
};

constexpr int kMaxCandidates = 8192;   // S / Bh limit of the selection sort
constexpr int kMaxTopK = 1024;
constexpr int kHistMaxEntries = 8192;  // (L / Bq) * k limit of the exact backward

// ---- launchers (host side; return hipSuccess or the launch error) --------
// K rows per (b, g): p.kv_rows; block i starts at row i * Bh + row_shift
// (full-sequence storage: row_shift 0).
hipError_t launch_summarize(const Prob& p, const void* k, int blk_begin,
                            int blk_end, float* summ, hipStream_t st, int row_shift = 0);
hipError_t launch_select(const Prob& p, const void* q, const float* summ,
                         int seg, int32_t* sel, hipStream_t st);
// Selection of segments seg0 .. seg0+nseg-1 in one launch.
hipError_t launch_select_pass(const Prob& p, const void* q, const float* summ, int seg0,
                              int nseg, int32_t* sel, hipStream_t st);
hipError_t launch_gather(const Prob& p, const void* k, const void* v,
                         const int32_t* sel, int seg, void* ko, void* vo,
                         hipStream_t st);
// With dO and delta given (bf16 only), the forward also writes the backward's
// row sums delta = rowsum(dO * o) into delta [B, Hq, L] (fused_delta returns
// whether it did); launch_bwd then skips its own delta pass (delta_ready).
bool fused_delta(const Prob& p);
hipError_t launch_fwd(const Prob& p, const void* q, const void* k,
                      const void* v, const int32_t* sel, int seg, void* o,
                      float* lse, hipStream_t st, const void* dO = nullptr,
                      float* delta = nullptr);
// Forward of segments seg0 .. seg0+nseg-1 in one launch (bf16 only; their
// selections must exist).  With dO, segment s's delta rows [B, Hq, L] go to
// delta + (s - seg0) * delta_stride bytes.
hipError_t launch_fwd_pass(const Prob& p, const void* q, const void* k, const void* v,
                           const int32_t* sel, int seg0, int nseg, void* o, float* lse,
                           hipStream_t st, const void* dO, float* delta, size_t delta_stride);
// hist_dk / hist_dv (exact gradient, bf16 only): fp32 [B, Hkv, S, D] sums
// of the gradient later segments gave each key; the backward adds them to
// its own rows and adds its queries' part to the history rows it selected.
hipError_t launch_bwd(const Prob& p, const void* q, const void* k,
                      const void* v, const void* o, const float* lse,
                      const void* dO, const int32_t* sel, int seg, void* dq,
                      void* dk, void* dv, float* delta_ws, hipStream_t st,
                      bool delta_ready = false, float* hist_dk = nullptr,
                      float* hist_dv = nullptr, float* partials = nullptr);
// Backward of segments seg0 .. seg0+nseg-1 in one dkdv and one dq launch
// (bf16 only; every segment's forward done, its delta rows [B, Hq, L] at
// delta + (s - seg0) * dstride bytes).
// With hist_dk / hist_dv (exact gradient): the fp32 sums later segments'
// queries left in the keys' rows are added to dk / dv.
hipError_t launch_bwd_pass(const Prob& p, const void* q, const void* k, const void* v,
                           const float* lse, const void* dO, const int32_t* sel, int seg0,
                           int nseg, void* dq, void* dk, void* dv, const float* delta,
                           size_t dstride, hipStream_t st, const float* hist_dk = nullptr,
                           const float* hist_dv = nullptr);
// Exact gradient over a whole pass: launch_hist_lists lists, for every
// segment 1 .. S/L-1 at once, the distinct history blocks its query blocks
// selected (into lists_ws, hist_lists_bytes); launch_hist_exact then adds
// segment seg's queries' dK/dV for those blocks into the fp32 sums hist_dk /
// hist_dv (segment seg's delta rows at delta_seg).
hipError_t launch_hist_lists(const Prob& p, const int32_t* sel, void* lists_ws,
                             hipStream_t st);
hipError_t launch_hist_exact(const Prob& p, const void* q, const void* k, const void* v,
                             const float* lse, const void* dO, const int32_t* sel, int seg,
                             const float* delta_seg, float* hist_dk, float* hist_dv,
                             void* lists_ws, hipStream_t st);
size_t hist_lists_bytes(const Prob& p);
// Stores zeros into n floats (n % 4 == 0, 16-byte aligned).
hipError_t launch_zero(float* p, size_t n, hipStream_t st);
size_t bwd_workspace_bytes(const Prob& p);
// Workspace parts of the backward: delta rows of one segment, and the dK/dV
// partial sums (launch_bwd's `partials`, else right after delta_ws).
size_t bwd_delta_bytes(const Prob& p);
size_t bwd_partial_bytes(const Prob& p);
size_t bwd_exact_workspace_bytes(const Prob& p);

// Decode step: selection of the n new tokens of q_new [B, Hq, n, D] (one
// unit, sel [B, Hkv, k]; scores: B*Hkv*nblk floats of scratch), then their
// attention (o [B, Hq, n, D], lse [B, Hq, n]) with the chunk partial sums
// in ws.  decode_score_ws points at the scores' part of the decode
// workspace, decode_cand_score_ws / decode_cand_idx_ws at the two-stage
// top-k's candidate lists (decode_cand_slots lists of k per (b, g)).
// decode_fused: the scoring launch also keeps each of its blocks' k best
// (score, index) pairs, and the history chunks of the attention launch pick
// the k best of those lists themselves (so no top-k launch runs between).
// decode_scoring_block: candidates per scoring block of a two-stage step
// with nb history blocks (128, or 256 when 128-candidate lists would leave
// more than 1,024 entries for the attention launch).
bool decode_fused(const Prob& p, int pos, int n);
int decode_cand_slots(const Prob& p);
int decode_scoring_block(const Prob& p, int nb);
float* decode_cand_score_ws(const Prob& p, void* ws);
int32_t* decode_cand_idx_ws(const Prob& p, void* ws);
hipError_t launch_select_decode(const Prob& p, const void* q_new, int n, int t0,
                                const float* summ, int32_t* sel, float* scores,
                                hipStream_t st, float* cand_score = nullptr,
                                int32_t* cand_idx = nullptr);
hipError_t launch_decode(const Prob& p, int pos, int n, const void* q_new, const void* k,
                         const void* v, int32_t* sel, void* o, float* lse, float* ws,
                         bool fused, hipStream_t st);
size_t decode_workspace_bytes(const Prob& p);
float* decode_score_ws(const Prob& p, void* ws);
int decode_max_rows();  // limit of G * n

// ---- host-RAM history tier (bf16) -----------------------------------------
// Window slots per (b, g): C = min(nqb * K, (S - L) / Bh) history blocks, the
// most one segment's query blocks can select together; window rows C*Bh + L.
int tier_slots(const Prob& p);
int tier_rows(const Prob& p);
// Segment seg: the union of the blocks its query blocks chose (sel), per
// (b, g) in ascending order -> list [B, Hkv, C] and count [B, Hkv]; wsel
// (the layout of sel) gets each entry's slot in that union, -1 kept.
hipError_t launch_tier_plan(const Prob& p, const int32_t* sel, int seg, int32_t* wsel,
                            int32_t* list, int32_t* count, hipStream_t st);
// Copies the listed blocks of the host K / V [B, Hkv, S, D] (device-mapped
// pinned memory) into window rows slot * Bh, and the segment's rows into
// window rows C * Bh .. C * Bh + L - 1 (window [B, Hkv, C*Bh + L, D]).
hipError_t launch_tier_fetch(const Prob& p, const void* k_host, const void* v_host,
                             const int32_t* list, const int32_t* count, int seg, void* kw,
                             void* vw, hipStream_t st);

// ---- profiling hooks (no-ops unless hga_profile_begin() was called) -----
// While kernel class kclass is profiled, returns true with a start / stop
// event pair for one launch (owned by the profiler until hga_profile_end).
bool prof_events(int kclass, hipEvent_t* start, hipEvent_t* stop);

}  // namespace hga

// Launches a kernel of class kc.  When that class is profiled, the dispatch
// itself stamps the start / stop events (hipExtLaunchKernelGGL), so timing
// adds no event packets, and no gaps, between kernels on the stream.
#define HGA_LAUNCH(kc, kern, grid, block, shm, st, ...)                                       \
  do {                                                                                        \
    hipEvent_t hga_ev0_ = nullptr, hga_ev1_ = nullptr;                                        \
    if (::hga::prof_events((kc), &hga_ev0_, &hga_ev1_))                                       \
      hipExtLaunchKernelGGL(kern, grid, block, shm, st, hga_ev0_, hga_ev1_, 0, __VA_ARGS__);  \
    else                                                                                      \
      hipLaunchKernelGGL(kern, grid, block, shm, st, __VA_ARGS__);                            \
  } while (0)

namespace hga {

}  // namespace hga

// ---------------------------------------------------------------------------
// Device helpers shared by the kernels
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)
namespace hga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// 8 bf16 packed in a uint4 -> 8 floats
__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
}

// Loads 16 bytes of T-typed data and widens them to floats (8 bf16 or 4 f32).
template <typename T> struct Vec16;
template <> struct Vec16<__bf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const __bf16* p, float* f) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    unpack_bf16x8(u, f);
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float* f) {
    float4 u = *reinterpret_cast<const float4*>(p);
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
  }
};

// Blocks of a 1-D grid are dealt round-robin over the 8 XCDs of the chip.
// Map the hardware block id to a work id so that consecutive work ids share
// an XCD (and therefore its L2): XCD x receives a contiguous range.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  int q = nblocks / kXcd, r = nblocks % kXcd;
  int x = bid % kXcd, slot = bid / kXcd;
  return (x < r) ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace hga
#endif
