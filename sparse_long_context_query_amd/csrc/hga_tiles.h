// Key/value tile staging and MFMA helpers shared by the HGA attention
// kernels (gfx950, bf16 in / fp32 accumulate).
//
// Key order of one query block ([JA] 背景と概要: a bounded exact set of
// history tokens plus the active segment): first the tokens of the selected
// history blocks, block after block in ascending block order, then the
// local tokens of the segment from its first token.  The kernels walk that
// order in tiles of TK (32 or 64) keys: history tiles over the concatenated
// selected blocks (the last one possibly partial), then local tiles starting
// at the segment start (causal masking per query).
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layout (64 lanes, lane = l, hi = l/32):
//   A (32 x 16): lane holds A[l%32][8*hi .. 8*hi+7]
//   B (16 x 32): lane holds B[8*hi .. 8*hi+7][l%32]
//   C (32 x 32): lane holds C[8*(r/4) + 4*hi + r%4][l%32], r = 0..15
// A product C = A.B contracting over an index that the other operand reads
// "down a column" needs that operand stored transposed.  Such tiles are
// staged into LDS transposed, with the 16-key groups permuted by swapping
// bits 2 and 3 of the key position: then the 8 k-values a lane feeds from
// an accumulator in C layout (rows 4*hi..4*hi+3 and 8+4*hi..8+4*hi+3 of a
// 16-row chunk) sit contiguously at positions 8*hi..8*hi+7.  Transposed
// rows are TK elements long with their 16-byte units XOR-swizzled by the
// row index to spread LDS banks.
#pragma once

#include "hga_internal.h"

namespace hga {

// position of key slot r inside a transposed row (swap bits 2 and 3)
__device__ __forceinline__ int tpos(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}
// Element offset of (row d, position pos) in a transposed TK-wide tile.
// 16-byte units of a row are XOR-swizzled so that the 8 consecutive rows a
// group of lanes reads in one go, and the rows one staging store touches,
// fall on different LDS banks.
template <int TK>
__device__ __forceinline__ int toff(int d, int pos) {
  static_assert(TK == 32 || TK == 64, "tile width");
  const int swz = (TK == 64) ? ((d + (d >> 3)) & 7) : (((d >> 1) + (d >> 3)) & 3);
  return d * TK + ((((pos >> 3) ^ swz) << 3) | (pos & 7));
}

template <int D, int TK>
struct TileGeom {
  static constexpr int KSTR = D + 8;           // row-major tile row stride (elements)
  static constexpr int ROW_ELEMS = TK * KSTR;   // one row-major tile
  static constexpr int T_ELEMS = D * TK;        // one transposed tile
  static constexpr int NJOB = (TK / 4) * (D / 8);  // jobs of 4 rows x 8 dims
};

__device__ __forceinline__ bf16x8 lds_b128(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Packs element e of four 8-wide rows into one 8-byte transposed quad.
__device__ __forceinline__ uint2 quad_column(const uint4& r0, const uint4& r1, const uint4& r2,
                                             const uint4& r3, int e) {
  auto pick = [e](const uint4& u) -> uint32_t {
    const uint32_t w = (e < 2) ? u.x : (e < 4) ? u.y : (e < 6) ? u.z : u.w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
  };
  return make_uint2(pick(r0) | (pick(r1) << 16), pick(r2) | (pick(r3) << 16));
}

// Where the keys of one query block come from: compacted list of selected
// history blocks (in LDS) followed by the local segment.
template <int TK>
struct KeySource {
  const int* hlist;  // selected block indices, valid entries only
  int nh;            // number of history tokens = count * Bh
  int Bh;
  int t0;            // segment start token
  int tend;          // one past the last local token of the segment
  int n_hist_tiles;  // ceil(nh / TK)

  __device__ __forceinline__ void init(const int* list, int count, int bh, int seg_start,
                                       int seg_end) {
    hlist = list;
    nh = count * bh;
    Bh = bh;
    t0 = seg_start;
    tend = seg_end;
    n_hist_tiles = (nh + TK - 1) / TK;
  }

  // first token of the 4-row group starting at tile row r4 of tile `it`,
  // or -1 if those rows hold no key.
  __device__ __forceinline__ int token4(int it, int r4) const {
    if (it < n_hist_tiles) {
      const int gs = it * TK + r4;
      if (gs >= nh) return -1;
      return hlist[gs / Bh] * Bh + gs % Bh;
    }
    const int t = t0 + (it - n_hist_tiles) * TK + r4;
    return t < tend ? t : -1;
  }
};

// Orders LDS traffic of one wave: its earlier LDS stores are visible to its
// later LDS loads from any lane (no other wave involved).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Compacts the valid entries (0 <= e < nb) of one selection row into LDS.
// Must be called by every thread of the block; returns the count.
__device__ __forceinline__ int compact_selection(const int32_t* __restrict__ row, int K, int nb,
                                                 int* hlist, int* count_slot) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int count = 0;
    for (int base = 0; base < K; base += 64) {
      const int e = (base + lane < K) ? row[base + lane] : -1;
      const bool ok = e >= 0 && e < nb;
      const unsigned long long m = __ballot(ok);
      const int pre = __popcll(m & ((1ull << lane) - 1ull));
      if (ok) hlist[count + pre] = e;
      count += __popcll(m);
    }
    if (lane == 0) *count_slot = count;
  }
  __syncthreads();
  return *count_slot;
}

}  // namespace hga
