// Host-RAM history tier (gfx950).
//
// The keys and values of the whole sequence live in pinned host memory;
// per segment only what its attention reads is brought into HBM: the
// history blocks its query blocks selected and the segment's own rows.
// This is the memory mechanism of the pages, applied per step, with the
// resident block summaries deciding what to move:
//   [JA] 背景と概要, [FR] Contexte: the history KV lives in system RAM and
//     only the active segment's state on the GPU;
//   [JA] 深掘り分析, [FR] Analyse approfondie: the block summaries stay
//     resident, and the limit moves from GPU memory to host capacity;
//   [JA] 今後の展望, [FR] Perspectives: the GPU-host transfers are the part
//     left to optimise.
//
// Two kernels, both driven by the selection on the GPU, so the host never
// waits for it:
//   plan:  per (b, g), the ascending union of the blocks chosen by the
//          segment's query blocks; each chosen block gets the slot of its rank
//          in that union, the selection is rewritten in slots (wsel, same
//          layout as sel) and the union is listed per slot;
//   fetch: copies the listed blocks into window rows slot * Bh and the
//          segment's own rows into window rows C * Bh .. C * Bh + L - 1,
//          reading the host memory directly (device-mapped pinned memory).
// Slots keep block order, so the attention kernels meet the same keys in the
// same order as with full-sequence storage.
#include <algorithm>

#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kRows = 16;         // window rows per copy unit
constexpr int kFetchBlocks = 32;   // blocks of the fetch grid
constexpr int kUnits = 2;          // copy units per block in flight

struct TierArgs {
  int nbg;          // B * Hkv
  int Hkv, Bh, L, K, nqb, nqb_all, seg, C;
  int nb;           // history blocks of the segment = seg * L / Bh
  int units_hist;   // C * Bh / kRows
  int units;        // units_hist + L / kRows
  int S, Sw;        // rows per (b, g): host storage, window
};

// One block of 256 threads per (b, g).
__global__ __launch_bounds__(256) void tier_plan_kernel(const int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ wsel,
                                                        int32_t* __restrict__ list,
                                                        int32_t* __restrict__ count,
                                                        TierArgs a) {
  __shared__ uint32_t bits[kMaxCandidates / 32];
  __shared__ int rank0[kMaxCandidates / 32];  // set bits in the words before
  __shared__ int wave_tot[4];
  const int bg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (a.nb + 31) / 32;  // <= 256
  for (int i = tid; i < nw; i += 256) bits[i] = 0u;
  __syncthreads();
  const size_t row0 = ((size_t)bg * a.nqb_all + (size_t)a.seg * a.nqb) * a.K;
  const int n = a.nqb * a.K;
  for (int i = tid; i < n; i += 256) {
    const int e = sel[row0 + i];
    if (e >= 0 && e < a.nb) atomicOr(&bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  // exclusive scan of the words' popcounts (one word per thread)
  const int c = tid < nw ? __popc(bits[tid]) : 0;
  int incl = c;
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  if (tid < nw) rank0[tid] = before + incl - c;
  __syncthreads();
  for (int i = tid; i < n; i += 256) {
    const int e = sel[row0 + i];
    int slot = -1;
    if (e >= 0 && e < a.nb)
      slot = rank0[e >> 5] + __popc(bits[e >> 5] & ((1u << (e & 31)) - 1u));
    wsel[row0 + i] = slot;
  }
  for (int w = tid; w < nw; w += 256) {
    uint32_t m = bits[w];
    int r = rank0[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      list[(size_t)bg * a.C + r++] = w * 32 + bit;
      m &= m - 1u;
    }
  }
  if (tid == 0) count[bg] = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
}

// Unit u of (b, g) is kRows rows of K and of V: history units first
// (slot = u * kRows / Bh; units of slots beyond the union's size are
// skipped), then the segment's own rows.  A small grid walks the units
// (grid stride, kUnits per pass of the loop, all their loads issued before
// the first store), which keeps enough requests in flight for the host
// link while it holds only a few CUs: the attention on the other stream
// needs every VGPR of the CUs it runs on.
template <int D>
__global__ __launch_bounds__(256) void tier_fetch_kernel(const __bf16* __restrict__ kh,
                                                         const __bf16* __restrict__ vh,
                                                         const int32_t* __restrict__ list,
                                                         const int32_t* __restrict__ count,
                                                         __bf16* __restrict__ kw,
                                                         __bf16* __restrict__ vw, TierArgs a) {
  constexpr int CH = kRows * D * 2 / 16;  // 16-byte chunks per tensor
  constexpr int PER = (2 * CH + 255) / 256;
  const int total = a.nbg * a.units;
  for (int w0 = blockIdx.x; w0 < total; w0 += kUnits * gridDim.x) {
    const uint4* src[kUnits][2];
    uint4* dst[kUnits][2];
    bool ok[kUnits];
#pragma unroll
    for (int n = 0; n < kUnits; ++n) {
      const int w = w0 + n * gridDim.x;
      ok[n] = w < total;
      if (!ok[n]) continue;
      const int bg = w / a.units;
      const int u = w % a.units;
      int src_row, dst_row;
      if (u < a.units_hist) {
        const int r = u * kRows;
        const int slot = r / a.Bh;
        ok[n] = slot < count[bg];
        if (!ok[n]) continue;
        src_row = list[(size_t)bg * a.C + slot] * a.Bh + r % a.Bh;
        dst_row = r;
      } else {
        const int r = (u - a.units_hist) * kRows;
        src_row = a.seg * a.L + r;
        dst_row = a.C * a.Bh + r;
      }
      src[n][0] = reinterpret_cast<const uint4*>(kh + ((size_t)bg * a.S + src_row) * D);
      src[n][1] = reinterpret_cast<const uint4*>(vh + ((size_t)bg * a.S + src_row) * D);
      dst[n][0] = reinterpret_cast<uint4*>(kw + ((size_t)bg * a.Sw + dst_row) * D);
      dst[n][1] = reinterpret_cast<uint4*>(vw + ((size_t)bg * a.Sw + dst_row) * D);
    }
    // every load first, then the stores: the host reads' latency is paid once
    uint4 x[kUnits][PER];
#pragma unroll
    for (int n = 0; n < kUnits; ++n) {
      if (!ok[n]) continue;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < 2 * CH) x[n][i] = c < CH ? src[n][0][c] : src[n][1][c - CH];
      }
    }
#pragma unroll
    for (int n = 0; n < kUnits; ++n) {
      if (!ok[n]) continue;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < 2 * CH) {
          if (c < CH) dst[n][0][c] = x[n][i];
          else dst[n][1][c - CH] = x[n][i];
        }
      }
    }
  }
}

TierArgs make_tier_args(const Prob& p, int seg) {
  TierArgs a;
  a.nbg = p.B * p.Hkv;
  a.Hkv = p.Hkv; a.Bh = p.Bh; a.L = p.L; a.K = p.K; a.nqb = p.nqb; a.nqb_all = p.nqb_all;
  a.seg = seg;
  a.C = tier_slots(p);
  a.nb = seg * p.L / p.Bh;
  a.units_hist = a.C * p.Bh / kRows;
  a.units = a.units_hist + p.L / kRows;
  a.S = p.S;
  a.Sw = a.C * p.Bh + p.L;
  return a;
}

}  // namespace

int tier_slots(const Prob& p) {
  const long long by_sel = (long long)p.nqb * p.K;
  const long long by_hist = (long long)(p.S - p.L) / p.Bh;
  return (int)(by_sel < by_hist ? by_sel : by_hist);
}

int tier_rows(const Prob& p) { return tier_slots(p) * p.Bh + p.L; }

hipError_t launch_tier_plan(const Prob& p, const int32_t* sel, int seg, int32_t* wsel,
                            int32_t* list, int32_t* count, hipStream_t st) {
  if (p.dtype != HGA_BF16 || p.Bh % kRows || p.L % kRows) return hipErrorInvalidValue;
  const TierArgs a = make_tier_args(p, seg);
  HGA_LAUNCH(HGA_K_TIER_PLAN, tier_plan_kernel, dim3(p.B * p.Hkv), dim3(256), 0, st, sel, wsel,
             list, count, a);
  return hipGetLastError();
}

hipError_t launch_tier_fetch(const Prob& p, const void* k_host, const void* v_host,
                             const int32_t* list, const int32_t* count, int seg, void* kw,
                             void* vw, hipStream_t st) {
  if (p.dtype != HGA_BF16 || p.Bh % kRows || p.L % kRows) return hipErrorInvalidValue;
  const TierArgs a = make_tier_args(p, seg);
  const dim3 grid(std::min(a.nbg * a.units, kFetchBlocks));
  if (p.D == 64)
    HGA_LAUNCH(HGA_K_TIER_FETCH, tier_fetch_kernel<64>, grid, dim3(256), 0, st,
               (const __bf16*)k_host, (const __bf16*)v_host, list, count, (__bf16*)kw,
               (__bf16*)vw, a);
  else
    HGA_LAUNCH(HGA_K_TIER_FETCH, tier_fetch_kernel<128>, grid, dim3(256), 0, st,
               (const __bf16*)k_host, (const __bf16*)v_host, list, count, (__bf16*)kw,
               (__bf16*)vw, a);
  return hipGetLastError();
}

}  // namespace hga
