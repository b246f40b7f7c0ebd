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
// Tiles are kept row-major in LDS (one key / query per row, 16-byte chunks
// XOR-swizzled per row).  An operand read along a row is one ds_read_b128;
// an operand read down a column (V^T, K^T, Q^T, dO^T) comes from two
// ds_read_b64_tr_b16.  A C-layout accumulator used as the next product's B
// operand supplies its 16 k-values in the order rows 4*hi..4*hi+3, then
// 8+4*hi..8+4*hi+3 of each 16-row group; the transposed reads fetch the
// other operand's rows in that same order.
#pragma once

#include "hga_internal.h"

namespace hga {

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
  int tpb;           // tiles per history block when Bh % TK == 0, else 0

  __device__ __forceinline__ void init(const int* list, int count, int bh, int seg_start,
                                       int seg_end) {
    hlist = list;
    nh = count * bh;
    Bh = bh;
    t0 = seg_start;
    tend = seg_end;
    n_hist_tiles = (nh + TK - 1) / TK;
    tpb = (bh % TK == 0) ? bh / TK : 0;
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

  // When every history tile lies inside one selected block (tpb > 0), the
  // rows of tile `it` are consecutive tokens: returns the (wave-uniform)
  // token of row 0, and row r is that plus r (local rows at or beyond the
  // segment end still map to t0 through local_row).
  __device__ __forceinline__ int tile_base(int it) const {
    if (it < n_hist_tiles) {
      const int bi = tpb == 1 ? it : it / tpb;
      const int blk = __builtin_amdgcn_readfirstlane(hlist[bi]);
      return blk * Bh + (it - bi * tpb) * TK;
    }
    return t0 + (it - n_hist_tiles) * TK;
  }
  __device__ __forceinline__ int contiguous_row(int it, int base, int r) const {
    const int t = base + r;
    return (it >= n_hist_tiles && t >= tend) ? t0 : t;
  }
};

// Walk order of the key tiles of KeySource for a block whose two halves share
// them out: the local tiles first (their rows are known before the selection
// has been read, so the first copies can start at once), then the history
// tiles; half h takes walk positions h, h + 2, h + 4, ...
__device__ __forceinline__ int walk_tile(int wpos, int nloc, int n_hist_tiles) {
  return wpos < nloc ? n_hist_tiles + wpos : wpos - nloc;
}

// Orders LDS traffic of one wave: its earlier LDS stores are visible to its
// later LDS loads from any lane (no other wave involved).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- row-major LDS tiles filled by direct global->LDS loads --------------
// A tile of bf16 rows of D elements is stored row-major without padding; the
// 16-byte chunk c of row r sits at chunk position c ^ swz<D>(r).  LDS serves
// 256 bytes per cycle, so the 16 rows a half-wave reads with ds_read_b128
// (same logical chunk) and the 4 rows x 4 chunks a half-wave reads with
// ds_read_b64_tr_b16 must land on 16 distinct 16-byte bank groups:
//   D = 128 (16 chunks per row): swz = 4*(r & 3) + ((r >> 2) & 3)
//   D =  64 (8 chunks, 2 rows per 256 bytes): swz = 4*((r >> 1) & 1) + ((r >> 2) & 3)
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int swz_byte(int r, int chunk) {
  return r * (2 * D) + ((chunk ^ swz<D>(r)) << 4);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ lds_void* to_lds(void* p) {
  return (lds_void*)(uintptr_t)(p);
}

// Raw buffer resource (stride 0) over `bytes` bytes at `base`.  Loads through
// it at byte offsets >= bytes return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes per lane from buffer byte offset `voff` straight into LDS at
// lds + 16*lane (buffer_load_dwordx4 ... lds; `lds` wave-uniform).  The
// buffer form is used rather than the global one: a global (FLAT-encoded)
// load into LDS still in flight makes the compiler's wait insertion drain
// every LDS read to lgkmcnt(0), which would serialise the MFMA operand reads
// of a double-buffered loop.  Tracked by vmcnt like any other vector load.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, to_lds(lds), 16, (int)voff, 0, 0, 0);
}

// One wave copies `rows` (a multiple of 1024/(2D)) bf16 rows of D elements,
// starting at global row pointer `g` (row stride D), into the swizzled
// tile at `lds` (wave-uniform), 1 KB per instruction, lane l writing
// bytes [16l, 16l+16) of each KB.  Rows at or beyond `valid` read row
// valid-1 instead (callers mask them); the buffer resource covers exactly
// the `valid` rows.  The data lands asynchronously: wait on vmcnt before
// reading.
template <int D>
__device__ __forceinline__ void dma_rows(const __bf16* g, int rows, int valid, unsigned char* lds,
                                         int lane) {
  constexpr int CPR = (2 * D) / 16;  // chunks per row
  constexpr int RPI = 64 / CPR;      // rows per 1 KB instruction
  const __amdgpu_buffer_rsrc_t r = make_rsrc(g, (uint32_t)valid * (2 * D));
  for (int i = 0; i < rows / RPI; ++i) {
    const int row = i * RPI + lane / CPR;
    const int p = lane % CPR;
    const int c = p ^ swz<D>(row);
    const int rr = row < valid ? row : valid - 1;
    buffer_to_lds16(r, (uint32_t)rr * (2 * D) + c * 16, lds + i * 1024);
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
// `kr` / `vr` cover the K and V rows of one (sequence, KV head).
template <int D, int TK>
__device__ __forceinline__ void dma_kv_tile(const KeySource<TK>& src, int it,
                                            __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                            unsigned char* kdst, unsigned char* vdst, int wr,
                                            int lane) {
  constexpr int CPR = (2 * D) / 16;
  constexpr int RPI = 64 / CPR;
  constexpr int NI = TK / RPI;
  static_assert(NI % 4 == 0, "instructions per wave");
  if (src.tpb > 0) {
    const int base = src.tile_base(it);
#pragma unroll
    for (int n = 0; n < NI / 4; ++n) {
      const int i = wr + 4 * n;
      const int row = i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz<D>(row);
      const uint32_t off = (uint32_t)src.contiguous_row(it, base, row) * (2 * D) + c * 16;
      buffer_to_lds16(kr, off, kdst + i * 1024);
      buffer_to_lds16(vr, off, vdst + i * 1024);
    }
    return;
  }
#pragma unroll
  for (int n = 0; n < NI / 4; ++n) {
    const int i = wr + 4 * n;
    const int row = i * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(row);
    const uint32_t off = (uint32_t)src.token_row(it, row) * (2 * D) + c * 16;
    buffer_to_lds16(kr, off, kdst + i * 1024);
    buffer_to_lds16(vr, off, vdst + i * 1024);
  }
}

// Split form of dma_kv_tile: the per-lane byte offsets of key tile `it`'s rows
// (branches allowed) and the issue of the copies (branch-free, so that it
// can be interleaved with other work).  A resource of 0 bytes (a tile that
// does not exist) turns the copies into loads of zeros from no memory.
template <int D, int TK>
__device__ __forceinline__ void kv_tile_offsets(const KeySource<TK>& src, int it, int wr,
                                                int lane, uint32_t (&off)[TK / (64 / ((2 * D) / 16)) / 4]) {
  constexpr int CPR = (2 * D) / 16;
  constexpr int RPI = 64 / CPR;
  constexpr int NI = TK / RPI;
  if (src.tpb > 0) {
    const int base = src.tile_base(it);
#pragma unroll
    for (int n = 0; n < NI / 4; ++n) {
      const int row = (wr + 4 * n) * RPI + lane / CPR;
      off[n] = (uint32_t)src.contiguous_row(it, base, row) * (2 * D) + ((lane % CPR) ^ swz<D>(row)) * 16;
    }
  } else {
#pragma unroll
    for (int n = 0; n < NI / 4; ++n) {
      const int row = (wr + 4 * n) * RPI + lane / CPR;
      off[n] = (uint32_t)src.token_row(it, row) * (2 * D) + ((lane % CPR) ^ swz<D>(row)) * 16;
    }
  }
}

// Lane byte offsets of kv_tile_offsets for a tile of consecutive rows
// starting at row 0 (loop-invariant; the tile's first row goes into the
// buffer resource instead).
template <int D, int TK>
__device__ __forceinline__ void contiguous_tile_offsets(int wr, int lane,
                                                        uint32_t (&off)[TK / (64 / ((2 * D) / 16)) / 4]) {
  constexpr int CPR = (2 * D) / 16;
  constexpr int RPI = 64 / CPR;
  constexpr int NI = TK / RPI;
#pragma unroll
  for (int n = 0; n < NI / 4; ++n) {
    const int row = (wr + 4 * n) * RPI + lane / CPR;
    off[n] = (uint32_t)row * (2 * D) + ((lane % CPR) ^ swz<D>(row)) * 16;
  }
}

template <int D, int TK>
__device__ __forceinline__ void kv_tile_issue(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                              const uint32_t (&off)[TK / (64 / ((2 * D) / 16)) / 4],
                                              unsigned char* kdst, unsigned char* vdst, int wr);

// dma_kv_tile with the scalar fast path: when every tile is a run of
// consecutive rows (tpb > 0) the lanes keep the fixed offsets `loff`
// (contiguous_tile_offsets) and the resource is placed at the tile's first
// row, over the rows up to the sequence end (rows past the segment end are
// read as they are; the kernels mask them).  k_rows / v_rows: row 0 of the
// (sequence, KV head), S rows.
template <int D, int TK>
__device__ __forceinline__ void dma_kv_tile_fast(
    const KeySource<TK>& src, int it, const __bf16* k_rows, const __bf16* v_rows, int S,
    __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
    const uint32_t (&loff)[TK / (64 / ((2 * D) / 16)) / 4], unsigned char* kdst,
    unsigned char* vdst, int wr, int lane) {
  if (src.tpb > 0) {
    const int base = src.tile_base(it);
    const uint32_t nbytes = (uint32_t)(S - base) * (2 * D);
    kv_tile_issue<D, TK>(make_rsrc(k_rows + (size_t)base * D, nbytes),
                         make_rsrc(v_rows + (size_t)base * D, nbytes), loff, kdst, vdst, wr);
  } else {
    dma_kv_tile<D, TK>(src, it, kr, vr, kdst, vdst, wr, lane);
  }
}

template <int D, int TK>
__device__ __forceinline__ void kv_tile_issue(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                              const uint32_t (&off)[TK / (64 / ((2 * D) / 16)) / 4],
                                              unsigned char* kdst, unsigned char* vdst, int wr) {
  constexpr int NI = TK / (64 / ((2 * D) / 16));
#pragma unroll
  for (int n = 0; n < NI / 4; ++n) {
    const int i = wr + 4 * n;
    buffer_to_lds16(kr, off[n], kdst + i * 1024);
    buffer_to_lds16(vr, off[n], vdst + i * 1024);
  }
}

// ds_read_b64_tr_b16 behind a restrict-qualified pointer.  Once inlined the
// read carries alias-scope metadata like any ordinary load, so the compiler's
// wait insertion treats it like the plain LDS reads beside it: it no longer
// waits for every direct global->LDS copy still in flight (those target the
// other buffer of a double-buffered pair; the copies a read depends on are
// waited for explicitly before the barrier that publishes them).
__device__ __forceinline__ bf16x4 lds_read_tr_b64(lds_bf16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
}

// Lane-constant byte offsets of the MFMA fragments inside a swizzled
// row-major tile of D-element bf16 rows, hoisted out of the tile loops.
// Moving by a multiple of 16 rows keeps swz() and only adds rows*2D bytes.
//   row fragment (tile row lq + 32*st, chunk 2kk+hi): rowf[kk] + st*32*2D
//   transposed fragment (tile rows rbase + 4hi + 0..3, then + 8..11, columns
//   of block db; rbase a multiple of 16): trf[db][0 / 1] + rbase*2D
template <int D>
struct FragOffsets {
  static constexpr int NKK = D / 16;
  static constexpr int NDB = D / 32;
  int rowf[NKK];
  int trf[NDB][2];
  __device__ __forceinline__ void init(int lane) {
    const int lq = lane & 31, hi = lane >> 5, j = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) rowf[kk] = swz_byte<D>(lq, 2 * kk + hi);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + 16 * (grp & 1) + 4 * (j & 3);
      const int r0 = 4 * hi + (j >> 2);
      trf[db][0] = swz_byte<D>(r0, d >> 3) + (d & 7) * 2;
      trf[db][1] = swz_byte<D>(r0 + 8, d >> 3) + (d & 7) * 2;
    }
  }
  __device__ __forceinline__ bf16x8 row(const unsigned char* tile, int st, int kk) const {
    return *reinterpret_cast<const bf16x8*>(tile + rowf[kk] + st * 32 * 2 * D);
  }
  __device__ __forceinline__ bf16x8 tr(const unsigned char* tile, int rbase, int db) const {
    const bf16x4 a = lds_read_tr_b64((lds_bf16x4*)to_lds((void*)(tile + trf[db][0] + rbase * 2 * D)));
    const bf16x4 b = lds_read_tr_b64((lds_bf16x4*)to_lds((void*)(tile + trf[db][1] + rbase * 2 * D)));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
};

// exp2 straight on v_exp_f32 (no denormal range fix-up: results below the
// normal range flush to zero, which the softmax never needs)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum of a value over the lane pair (l, l^32) that holds one query's
// two halves of a C-layout column: v_permlane32_swap, a VALU op (no LDS).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
