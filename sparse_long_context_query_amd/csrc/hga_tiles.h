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

  // token of row r of tile `it`; rows that hold no key map to the segment's
  // first token (a valid row whose scores the kernels mask).
  __device__ __forceinline__ int token_row(int it, int r) const {
    if (it < n_hist_tiles) {
      const int gs = it * TK + r;
      return gs < nh ? hlist[gs / Bh] * Bh + gs % Bh : t0;
    }
    const int t = t0 + (it - n_hist_tiles) * TK + r;
    return t < tend ? t : t0;
  }
};


// Orders LDS traffic of one wave: its earlier LDS stores are visible to its
// later LDS loads from any lane (no other wave involved).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- row-major LDS tiles filled by direct global->LDS loads --------------
// A tile of bf16 rows of D elements is stored row-major without padding; the
// 16-byte chunk c of row r sits at chunk position c ^ sw8(r), which puts
// the 8 rows a group of lanes reads at once (and the 4 rows of a transposed
// read) on distinct LDS banks.
__device__ __forceinline__ int sw8(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

template <int D>
__device__ __forceinline__ int swz_byte(int r, int chunk) {
  return r * (2 * D) + ((chunk ^ sw8(r)) << 4);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ lds_void* to_lds(void* p) {
  return (lds_void*)(uintptr_t)(p);
}

// One wave copies `rows` (a multiple of 1024/(2D)) bf16 rows of D elements,
// starting at global row pointer `g` (row stride D), into the swizzled
// tile at `lds` (wave-uniform), 1 KB per instruction, lane l writing
// bytes [16l, 16l+16) of each KB.  Rows at or beyond `valid` read row
// valid-1 instead (callers mask them), so every global address stays in
// bounds.  The data lands asynchronously: wait on vmcnt before reading.
template <int D>
__device__ __forceinline__ void dma_rows(const __bf16* g, int rows, int valid, unsigned char* lds,
                                         int lane) {
  constexpr int CPR = (2 * D) / 16;  // chunks per row
  constexpr int RPI = 64 / CPR;      // rows per 1 KB instruction
  for (int i = 0; i < rows / RPI; ++i) {
    const int row = i * RPI + lane / CPR;
    const int p = lane % CPR;
    const int c = p ^ sw8(row);
    const int rr = row < valid ? row : valid - 1;
    __builtin_amdgcn_global_load_lds((const void*)(g + (size_t)rr * D + c * 8),
                                     to_lds(lds + i * 1024), 16, 0, 0);
  }
}

// Transposed 32x16 A-operand fragment from a swizzled row-major tile: the
// MFMA rows are the tile's columns d in [32*db, 32*db+32), the 16 k-values
// are tile rows rbase + {4hi..4hi+3, 8+4hi..8+4hi+3} (the same 16-row
// permutation the C-layout B operands use).  Two ds_read_b64_tr_b16: in each
// group of 16 lanes, lane j receives element j%4 of the 8-byte pieces read
// by lanes j/4, j/4+4, j/4+8, j/4+12; lane i points at tile row
// rbase+4hi(+8)+i/4, columns 32db+16*(group&1)+4*(i%4) .. +3.
template <int D>
__device__ __forceinline__ bf16x8 tr_fragment(const unsigned char* tile, int rbase, int db,
                                              int lane) {
  const int j = lane & 15, grp = lane >> 4, hi = lane >> 5;
  const int d = 32 * db + 16 * (grp & 1) + 4 * (j & 3);
  const int chunk = d >> 3, boff = (d & 7) * 2;
  const int r0 = rbase + 4 * hi + (j >> 2);
  const int r1 = r0 + 8;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)to_lds((void*)(tile + swz_byte<D>(r0, chunk) + boff)));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)to_lds((void*)(tile + swz_byte<D>(r1, chunk) + boff)));
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Row-major A/B-operand fragment: row r, elements 16kk+8hi .. +7.
template <int D>
__device__ __forceinline__ bf16x8 row_fragment(const unsigned char* tile, int r, int kk, int hi) {
  return *reinterpret_cast<const bf16x8*>(tile + swz_byte<D>(r, 2 * kk + hi));
}

// The 4 waves of one half of a block of threads copy the K and V rows of
// key tile `it` straight into swizzled row-major LDS tiles (one 1 KB
// direct load per wave and instruction, every lane supplying its own row).
template <int D, int TK>
__device__ __forceinline__ void dma_kv_tile(const KeySource<TK>& src, int it, const __bf16* kg,
                                            const __bf16* vg, unsigned char* kdst,
                                            unsigned char* vdst, int wr, int lane) {
  constexpr int CPR = (2 * D) / 16;
  constexpr int RPI = 64 / CPR;
  constexpr int NI = TK / RPI;
  static_assert(NI % 4 == 0, "instructions per wave");
#pragma unroll
  for (int n = 0; n < NI / 4; ++n) {
    const int i = wr + 4 * n;
    const int row = i * RPI + lane / CPR;
    const int c = (lane % CPR) ^ sw8(row);
    const size_t off = (size_t)src.token_row(it, row) * D + c * 8;
    __builtin_amdgcn_global_load_lds((const void*)(kg + off), to_lds(kdst + i * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(vg + off), to_lds(vdst + i * 1024), 16, 0, 0);
  }
}

// Lane-constant byte offsets of the MFMA fragments inside a swizzled
// row-major tile of D-element bf16 rows, hoisted out of the tile loops.
// Moving by a multiple of 8 rows keeps sw8() and only adds rows*2D bytes;
// chunks c and c+8 of a row differ by 128 bytes after the swizzle.  So:
//   row fragment (row lq + 32*st, chunk 2kk+hi):
//       rowf[kk & 3] + (kk >> 2) * 128 + st * 32 * 2D
//   transposed fragment (tile rows rbase + 4hi.. (+8), columns of block db):
//       first read  trf[db & 1] + (db >> 1) * 128 + rbase * 2D
//       second read the same + 8 * 2D
template <int D>
struct FragOffsets {
  int rowf[4];
  int trf[2];
  __device__ __forceinline__ void init(int lane) {
    const int lq = lane & 31, hi = lane >> 5, j = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) rowf[kk] = swz_byte<D>(lq, 2 * kk + hi);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = 32 * db + 16 * (grp & 1) + 4 * (j & 3);
      trf[db] = swz_byte<D>(4 * hi + (j >> 2), d >> 3) + (d & 7) * 2;
    }
  }
  __device__ __forceinline__ bf16x8 row(const unsigned char* tile, int st, int kk) const {
    return *reinterpret_cast<const bf16x8*>(tile + rowf[kk & 3] + (kk >> 2) * 128 +
                                            st * 32 * 2 * D);
  }
  __device__ __forceinline__ bf16x8 tr(const unsigned char* tile, int rbase, int db) const {
    const unsigned char* p = tile + trf[db & 1] + (db >> 1) * 128 + rbase * 2 * D;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)to_lds((void*)p));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)to_lds((void*)(p + 8 * 2 * D)));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
};

// exp2 straight on v_exp_f32 (no denormal range fix-up: results below the
// normal range flush to zero, which the softmax never needs)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Waits for every outstanding vector-memory load of this wave (vmcnt(0);
// expcnt and lgkmcnt left at their maxima).  Used once before a pipelined
// loop so that operands loaded ahead of it do not make the compiler wait
// for in-flight prefetches inside the loop.
__device__ __forceinline__ void drain_vmem_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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
