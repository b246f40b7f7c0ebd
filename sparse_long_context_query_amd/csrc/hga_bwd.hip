// a6 + a7 + a8: HGA backward of one segment with history detached, gfx950.
//
// [FR] Analyse approfondie: only the active segment's gradients are computed
// and kept on the GPU; the KV states of earlier segments leave the graph
// ([FR] Contexte: they are decoupled from the differentiable state).  So
// the selected history keys feed dq but receive no gradient, and the
// selection itself is not differentiated.  For the loss with dL/do = dO:
//   delta_t = sum_d dO[t,d] o[t,d]
//   p_ti    = exp(scale q_t.k_i - lse_t)
//   dS_ti   = p_ti (dO_t.v_i - delta_t)
//   dq_t    = scale sum_i dS_ti k_i                 (history + local keys)
//   dk_i    = scale sum_t dS_ti q_t,  dv_i = sum_t p_ti dO_t
//             (local keys i only; t runs over the segment's queries that see
//              key i and over the G query heads of its KV head)
// Three kernels: delta (row reduction), dq (parallel over query rows, walks
// the same key tiles as the forward) and dk/dv (parallel over local key
// tiles, walks the causal query tiles of every head of the group); no
// floating-point atomics, so results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "hga_internal.h"
#include "hga_tiles.h"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
  int B, S, L, Bh, Bq, K, Hq, Hkv, G, nqb, nqb_all, seg;
  // whole-pass launches: segments seg .. seg+nseg-1; segment s's delta rows
  // sit (s - seg) * dchunk floats further on
  int nseg;
  int dchunk;
  int wpu;      // dq: blocks of threads per (b, g, j) unit
  int nq32;     // 32-row query sub-blocks per query block
  float c2;     // scale * log2(e)
  float scale;
  // exact-gradient backward only (else null): fp32 [B, Hkv, S, D] sums of
  // the gradient that later segments' queries gave each key (dK scaled)
  float* hdk;
  float* hdv;
  int Skv;    // step kernels: K/V rows per (b, g)
  int kv_t0;  // step kernels: K/V row of the segment's first key
};

// ---------------------------------------------------------------------------
// a6: delta[b,h,t-t0] = sum_d dO*o, 16 lanes per row, fp32.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o,
                                                    const T* __restrict__ dO,
                                                    float* __restrict__ delta, int S, int L,
                                                    int t0, int nrows) {
  constexpr int E = Vec16<T>::N;
  constexpr int C = D / E;     // lanes per row
  constexpr int RPB = 256 / C;  // rows per block of threads
  const int row = blockIdx.x * RPB + threadIdx.x / C;
  const int c = threadIdx.x % C;
  float s = 0.f;
  if (row < nrows) {
    const int bh = row / L, t = row % L;
    const size_t off = ((size_t)bh * S + t0 + t) * D + c * E;
    float x[E], y[E];
    Vec16<T>::load(o + off, x);
    Vec16<T>::load(dO + off, y);
#pragma unroll
    for (int e = 0; e < E; ++e) s += x[e] * y[e];
  }
#pragma unroll
  for (int m = C / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, C);
  if (row < nrows && c == 0) delta[row] = s;
}

// Fixed cost of one dkdv item (K/V copy, fold, stores) in units of the cost
// of one (head, query tile) pair, measured at D = 128: the block that runs
// two items gets that many fewer pairs.
constexpr int kDkdvItemCost = 16;

// Pairs of key tile p (of nkt) that block 2p takes; the rest of tile p, if
// any, goes to block 2p+1 ahead of the mirror tile's wl pairs.  When the
// result is below wh = G*(nkt-p), tile p is left as two fp32 partial sums.
__device__ __forceinline__ int dkdv_split(int wh, int wl) {
  if (wl == 0) return (wh + 1) >> 1;
  const int s = (wh + wl + kDkdvItemCost + 1) >> 1;
  return s < wh ? s : wh;
}
__device__ __forceinline__ int dkdv_mirror_pairs(int p, int nkt, int G) {
  return p < (nkt >> 1) ? G * (p + 1) : 0;  // tiles below nkt/2 have a mirror
}

// Last step of a8 for the key tiles whose dk/dv work two dkdv blocks shared:
// adds the two fp32 partial sums in a fixed order (part 0 + part 1), scales
// dK and rounds to bf16.  Runs in the kernel launched right after the dkdv
// kernel (the launch boundary makes the partial sums visible); the work is
// strided over all of its threads, one item = 4 consecutive elements of one
// key row of one slot.
template <int D>
__device__ __forceinline__ void dkdv_finish(const float* __restrict__ part_ws,
                                            __bf16* __restrict__ dk, __bf16* __restrict__ dv,
                                            const BwdArgs& a, int nph) {
  constexpr int C4 = D / 4;
  const int nkt = (a.L + 31) / 32;
  const int total = a.B * a.Hkv * nph * 32 * C4;
  const int t0 = a.seg * a.L;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int c4 = i % C4;
    const int key = (i / C4) % 32;
    const int rest = i / (C4 * 32);
    const int slot = rest % nph;
    const int bg = rest / nph;
    const int tk = t0 + slot * 32 + key;
    if (tk >= t0 + a.L) continue;
    const int wh = a.G * (nkt - slot);  // pairs of key tile `slot`
    if (dkdv_split(wh, dkdv_mirror_pairs(slot, nkt, a.G)) >= wh) continue;
    const float* p0 = part_ws + ((size_t)(bg * nph + slot) * 2) * 64 * D;
    const float* p1 = p0 + 64 * D;
    const float4 ka = reinterpret_cast<const float4*>(p0 + (size_t)key * D)[c4];
    const float4 kb = reinterpret_cast<const float4*>(p1 + (size_t)key * D)[c4];
    const float4 va = reinterpret_cast<const float4*>(p0 + (size_t)(32 + key) * D)[c4];
    const float4 vb = reinterpret_cast<const float4*>(p1 + (size_t)(32 + key) * D)[c4];
    const size_t off = ((size_t)bg * a.S + tk) * D + 4 * c4;
    float4 hk = make_float4(0.f, 0.f, 0.f, 0.f), hv = hk;
    if (a.hdk != nullptr) {  // exact gradient: what later segments added
      hk = *reinterpret_cast<const float4*>(a.hdk + off);
      hv = *reinterpret_cast<const float4*>(a.hdv + off);
    }
    const bf16x4 ko = {(__bf16)((ka.x + kb.x) * a.scale + hk.x),
                       (__bf16)((ka.y + kb.y) * a.scale + hk.y),
                       (__bf16)((ka.z + kb.z) * a.scale + hk.z),
                       (__bf16)((ka.w + kb.w) * a.scale + hk.w)};
    const bf16x4 vo = {(__bf16)(va.x + vb.x + hv.x), (__bf16)(va.y + vb.y + hv.y),
                       (__bf16)(va.z + vb.z + hv.z), (__bf16)(va.w + vb.w + hv.w)};
    *reinterpret_cast<bf16x4*>(dk + off) = ko;
    *reinterpret_cast<bf16x4*>(dv + off) = vo;
  }
}

// ---------------------------------------------------------------------------
// a7, bf16 MFMA: dq.  Same work split as the forward: 512 threads = 8 waves,
// up to 4 wave rows (32 queries of one head each) of one (b, g, j) unit per
// block of threads; the key tiles (64 keys) are dealt alternately to two
// halves, waves 0-3 and 4-7, local tiles first (walk_tile), each half
// double-buffering swizzled row-major K and V tiles that are copied straight
// from memory into LDS.  Per wave and 32-key sub-tile:
//   S^T  = K . Q^T          (Q^T in registers as B operand)
//   dP^T = V . dO^T         (dO^T in registers as B operand)
//   dS^T = P^T * (dP^T - delta),  P^T = exp2(S^T c2 - lse2)
//   dQ^T += K^T . dS^T      (K^T read transposed from the K tile, dS^T
//                            straight from the accumulator)
// The two halves' partial dQ^T are added through LDS at the end.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512) void dq_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    const int32_t* __restrict__ sel, __bf16* __restrict__ dq, const float* __restrict__ part_ws,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, int nph, BwdArgs a) {
  constexpr int TK = 64;
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE_B = TK * 2 * D;
  constexpr int STAGE_B = 2 * TILE_B;  // K tile + V tile
  static_assert(4 * STAGE_B >= 4 * NDB * 16 * 64 * 4, "merge buffer fits");

  __shared__ __attribute__((aligned(1024))) unsigned char s_tiles[2][2][STAGE_B];  // [half][buf]
  __shared__ int s_hlist[kMaxTopK];
  __shared__ int s_hcount;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int c = w % a.wpu;
  const int j = (w / a.wpu) % a.nqb;
  const int g = (w / (a.wpu * a.nqb)) % a.Hkv;
  const int b = w / (a.wpu * a.nqb * a.Hkv);
  const int t0 = a.seg * a.L;
  const int nb = t0 / a.Bh;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63, lq = lane & 31, hi = lane >> 5;
  const int half = wave >> 2, wr = wave & 3;

  const int nwr = a.G * a.nq32;
  const int idx = c * 4 + wr;
  const bool active = idx < nwr;
  const int qs = idx / a.G, hh = idx % a.G;
  const int h = g * a.G + hh;
  const int qfirst = t0 + j * a.Bq + qs * 32;
  const int nvalid = active ? min(32, a.Bq - qs * 32) : 0;
  const int wave_qmax = qfirst + nvalid - 1;
  int blk_qmax = t0;
  for (int ww = 0; ww < 4; ++ww) {
    const int id2 = c * 4 + ww;
    if (id2 < nwr) {
      const int q2 = id2 / a.G;
      blk_qmax = max(blk_qmax, t0 + j * a.Bq + q2 * 32 + min(32, a.Bq - q2 * 32) - 1);
    }
  }

  // the first local tile's copies and the query-side rows do not depend on
  // the selection: request them first so that their latency overlaps the
  // partial-sum finish and the compaction (local tiles come first in the
  // walk order)
  const int nloc = (blk_qmax - t0) / TK + 1;  // local tiles any wave of the block sees
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.Skv * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kv_base, (uint32_t)a.Skv * (2 * D));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + kv_base, (uint32_t)a.Skv * (2 * D));
  if (half < nloc) {
    KeySource<TK> loc;
    loc.init(s_hlist, 0, a.Bh, a.kv_t0, a.kv_t0 + a.L);  // K/V rows, not tokens
    dma_kv_tile<D, TK>(loc, half, kr, vr, s_tiles[half][0], s_tiles[half][0] + TILE_B, wr, lane);
  }
  const int tq = qfirst + lq;
  const bool row_ok = lq < nvalid;
  const size_t qrow = (size_t)(b * a.Hq + h) * a.S + tq;
  bf16x8 qreg[NKK], doreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qreg[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(q + qrow * D + 16 * kk + 8 * hi) : bf16x8{};
    doreg[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(dO + qrow * D + 16 * kk + 8 * hi) : bf16x8{};
  }
  const float lse2 = row_ok ? lse[qrow] * kLog2e : 0.f;
  const float dlt = row_ok ? delta[(size_t)(b * a.Hq + h) * a.L + (tq - t0)] : 0.f;

  dkdv_finish<D>(part_ws, dk, dv, a, nph);

  const int32_t* srow = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)a.seg * a.nqb + j) * a.K;
  const int nsel = compact_selection(srow, a.K, nb, s_hlist, &s_hcount);
  KeySource<TK> src;
  src.init(s_hlist, nsel, a.Bh, a.kv_t0, a.kv_t0 + a.L);
  const int ntiles = src.n_hist_tiles + nloc;
  const int n0 = (ntiles + 1) / 2;  // walk positions of half 0; half 1 has ntiles - n0
  const int nht = src.n_hist_tiles;


  floatx16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = floatx16{};
  floatx16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = -dlt;
  FragOffsets<D> fo;
  fo.init(lane);

  if (half >= nloc && half < ntiles)  // a history tile first: after the compaction
    dma_kv_tile<D, TK>(src, walk_tile(half, nloc, nht), kr, vr, s_tiles[half][0],
                       s_tiles[half][0] + TILE_B, wr, lane);
  drain_vmem_loads();
  __syncthreads();

  for (int i = 0; i < n0; ++i) {
    const int wpos = 2 * i + half;
    const bool mine = wpos < ntiles;
    const int it = walk_tile(mine ? wpos : half, nloc, nht);
    if (wpos + 2 < ntiles)
      dma_kv_tile<D, TK>(src, walk_tile(wpos + 2, nloc, nht), kr, vr, s_tiles[half][(i + 1) & 1],
                         s_tiles[half][(i + 1) & 1] + TILE_B, wr, lane);
    const bool is_local = it >= src.n_hist_tiles;
    const int local_first = t0 + (it - src.n_hist_tiles) * TK;
    const bool work = mine && active && (!is_local || local_first <= wave_qmax);
    if (work) {
      const unsigned char* kt = s_tiles[half][i & 1];
      const unsigned char* vt = kt + TILE_B;
      const int base = is_local ? local_first : it * TK;
      const int lim = is_local ? tq : src.nh - 1;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (is_local && local_first + 32 * st > wave_qmax) break;  // sub-tile fully masked
        // K and V fragments of the sub-tile are requested well ahead of their
        // MFMAs (the LDS latency is not paid once per k-step)
        bf16x8 kf[NKK], vf[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          kf[kk] = fo.row(kt, st, kk);
          vf[kk] = fo.row(vt, st, kk);
        }
        // dP starts from -delta (constant along a lane, the query), so the
        // products give dP - delta directly
        floatx16 sacc = floatx16{}, pacc = negd;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sacc = mfma32(kf[kk], qreg[kk], sacc);
          pacc = mfma32(vf[kk], doreg[kk], pacc);
        }
        // software pipeline 8 fragments deep: 8 reads, then 2 MFMAs per 2
        // further reads, then the last 8 MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int u = 0; u < NKK - 4; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        const bool need_mask = is_local ? (local_first + 32 * st + 31 > qfirst)
                                        : ((it * TK + 32 * st + 32) > src.nh);
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr_ = base + 32 * st + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (kr_ > lim) sacc[r] = -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[r], a.c2, -lse2));
          sacc[r] = p * pacc[r];
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 8 * ks;
          const bf16x8 sb = to_bf16x8(sacc[r0], sacc[r0 + 1], sacc[r0 + 2], sacc[r0 + 3],
                                      sacc[r0 + 4], sacc[r0 + 5], sacc[r0 + 6], sacc[r0 + 7]);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            dqacc[db] = mfma32(fo.tr(kt, 32 * st + 16 * ks, db), sb, dqacc[db]);
        }
      }
    }
    drain_vmem_loads();
    __syncthreads();
  }

  // add the two halves' partial dQ^T through LDS, scale, round, store
  float4* park = reinterpret_cast<float4*>(&s_tiles[0][0][0]) + wr * (NDB * 4 * 64);
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        park[(db * 4 + r4) * 64 + lane] = make_float4(dqacc[db][4 * r4], dqacc[db][4 * r4 + 1],
                                                      dqacc[db][4 * r4 + 2], dqacc[db][4 * r4 + 3]);
  }
  __syncthreads();
  if (half == 0 && active && row_ok) {
    __bf16* op = dq + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 p4 = park[(db * 4 + r4) * 64 + lane];
        const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = (__bf16)((dqacc[db][4 * r4 + e] + pv[e]) * a.scale);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * r4 + 4 * hi) = pk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// a7, bf16 MFMA, whole segmented pass: dq of segments a.seg .. a.seg+a.nseg-1
// in one launch.  As fwd_pass_kernel: a block of 4 waves owns up to 4 wave
// rows of one (segment, b, g, j) unit and walks every key tile of the unit
// itself (local tiles first, then history), two blocks per CU with no
// common barrier, no halves to add at the end; same work order (contiguous
// (b, g) ranges per XCD, last segments and query blocks first).  Per wave
// and 32-key sub-tile the products are those of dq_bf16_kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void dq_pass_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    const int32_t* __restrict__ sel, __bf16* __restrict__ dq, BwdArgs a) {
  constexpr int TK = 64;
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE_B = TK * 2 * D;
  constexpr int STAGE_B = 2 * TILE_B;  // K tile + V tile

  __shared__ __attribute__((aligned(1024))) unsigned char s_tiles[2][STAGE_B];
  __shared__ int s_hlist[kMaxTopK];
  __shared__ int s_hcount;

  int w = xcd_remap(blockIdx.x, gridDim.x);
  const int c = w % a.wpu;
  w /= a.wpu;
  const int j = a.nqb - 1 - w % a.nqb;
  w /= a.nqb;
  const int sg = a.nseg - 1 - w % a.nseg;
  w /= a.nseg;
  const int g = w % a.Hkv;
  const int b = w / a.Hkv;
  const int seg = a.seg + sg;
  const int t0 = seg * a.L;
  const int nb = t0 / a.Bh;

  const int tid = threadIdx.x;
  const int wr = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63, lq = lane & 31, hi = lane >> 5;

  const int nwr = a.G * a.nq32;
  const int idx = c * 4 + wr;
  const bool active = idx < nwr;
  const int qs = idx / a.G, hh = idx % a.G;
  const int h = g * a.G + hh;
  const int qfirst = t0 + j * a.Bq + qs * 32;
  const int nvalid = active ? min(32, a.Bq - qs * 32) : 0;
  const int wave_qmax = qfirst + nvalid - 1;
  int blk_qmax = t0;
  for (int ww = 0; ww < 4; ++ww) {
    const int id2 = c * 4 + ww;
    if (id2 < nwr) {
      const int q2 = id2 / a.G;
      blk_qmax = max(blk_qmax, t0 + j * a.Bq + q2 * 32 + min(32, a.Bq - q2 * 32) - 1);
    }
  }

  // the first local tile's copies and the query-side rows do not depend on
  // the selection: request them first, so that their latency overlaps the
  // compaction
  const int nloc = (blk_qmax - t0) / TK + 1;
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kv_base, (uint32_t)a.S * (2 * D));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + kv_base, (uint32_t)a.S * (2 * D));
  uint32_t loff[TK / (64 / ((2 * D) / 16)) / 4];
  contiguous_tile_offsets<D, TK>(wr, lane, loff);
  {
    KeySource<TK> loc;
    loc.init(s_hlist, 0, a.Bh, t0, t0 + a.L);
    dma_kv_tile_fast<D, TK>(loc, 0, k + kv_base, v + kv_base, a.S, kr, vr, loff, s_tiles[0],
                            s_tiles[0] + TILE_B, wr, lane);
  }
  const int tq = qfirst + lq;
  const bool row_ok = lq < nvalid;
  const size_t qrow = (size_t)(b * a.Hq + h) * a.S + tq;
  bf16x8 qreg[NKK], doreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qreg[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(q + qrow * D + 16 * kk + 8 * hi) : bf16x8{};
    doreg[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(dO + qrow * D + 16 * kk + 8 * hi) : bf16x8{};
  }
  const float lse2 = row_ok ? lse[qrow] * kLog2e : 0.f;
  const float dlt =
      row_ok ? delta[(size_t)sg * a.dchunk + (size_t)(b * a.Hq + h) * a.L + (tq - t0)] : 0.f;

  const int32_t* srow = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)seg * a.nqb + j) * a.K;
  const int nsel = compact_selection(srow, a.K, nb, s_hlist, &s_hcount);
  KeySource<TK> src;
  src.init(s_hlist, nsel, a.Bh, t0, t0 + a.L);
  const int nht = src.n_hist_tiles;
  const int ntiles = nht + nloc;

  floatx16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = floatx16{};
  floatx16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = -dlt;
  FragOffsets<D> fo;
  fo.init(lane);
  drain_vmem_loads();
  __syncthreads();

  for (int i = 0; i < ntiles; ++i) {
    const int it = walk_tile(i, nloc, nht);
    if (i + 1 < ntiles)
      dma_kv_tile_fast<D, TK>(src, walk_tile(i + 1, nloc, nht), k + kv_base, v + kv_base, a.S,
                              kr, vr, loff, s_tiles[(i + 1) & 1], s_tiles[(i + 1) & 1] + TILE_B,
                              wr, lane);
    const bool is_local = it >= nht;
    const int local_first = t0 + (it - nht) * TK;
    const bool work = active && (!is_local || local_first <= wave_qmax);
    if (work) {
      const unsigned char* kt = s_tiles[i & 1];
      const unsigned char* vt = kt + TILE_B;
      const int base = is_local ? local_first : it * TK;
      const int lim = is_local ? tq : src.nh - 1;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (is_local && local_first + 32 * st > wave_qmax) break;  // sub-tile fully masked
        bf16x8 kf[NKK], vf[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          kf[kk] = fo.row(kt, st, kk);
          vf[kk] = fo.row(vt, st, kk);
        }
        // dP starts from -delta (constant along a lane, the query), so the
        // products give dP - delta directly
        floatx16 sacc = floatx16{}, pacc = negd;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sacc = mfma32(kf[kk], qreg[kk], sacc);
          pacc = mfma32(vf[kk], doreg[kk], pacc);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int u = 0; u < NKK - 4; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        const bool need_mask = is_local ? (local_first + 32 * st + 31 > qfirst)
                                        : ((it * TK + 32 * st + 32) > src.nh);
        if (need_mask) {
          // a fence with side effects keeps this a branch: if-converted, the
          // selects would run on every tile
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr_ = base + 32 * st + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (kr_ > lim) sacc[r] = -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[r], a.c2, -lse2));
          sacc[r] = p * pacc[r];
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 8 * ks;
          const bf16x8 sb = to_bf16x8(sacc[r0], sacc[r0 + 1], sacc[r0 + 2], sacc[r0 + 3],
                                      sacc[r0 + 4], sacc[r0 + 5], sacc[r0 + 6], sacc[r0 + 7]);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            dqacc[db] = mfma32(fo.tr(kt, 32 * st + 16 * ks, db), sb, dqacc[db]);
        }
      }
    }
    drain_vmem_loads();
    __syncthreads();
  }

  if (!(active && row_ok)) return;
  __bf16* op = dq + qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(dqacc[db][4 * r4 + e] * a.scale);
      *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * r4 + 4 * hi) = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// a8, bf16 MFMA: dk/dv of the local keys.  The work of a 32-key tile kt is
// its (query head, 32-query tile) pairs: query tiles kt.. of every head of
// the group, G*(nqt-kt) of them, so causality makes early key tiles up to
// nqt times heavier than late ones.  Blocks are balanced by pairing key tile
// p with its mirror nqt-1-p: their combined pairs are split between block 2p
// (first part of tile p) and block 2p+1 (rest of tile p, then the whole
// mirror tile), the latter taking kDkdvItemCost fewer pairs for its second
// item.  When tile p is split, both blocks publish fp32 partial sums of it in
// the workspace, and the dq kernel, launched next in the same backward call,
// adds them in a fixed order and writes the rows (dkdv_finish).  Other tiles
// are written directly.
//
// Per item (one key tile and a range of its pairs) the pairs are dealt
// round-robin to the 8 waves, two per SIMD, so one wave's loads and softmax
// overlap the other's MFMAs.  A wave copies its pair's Q and dO tiles and
// their lse / delta straight from memory into its own swizzled LDS slice (no
// register staging), then, with the key tile's K and V rows in LDS:
//   S  = Q . K^T,  dP = dO . V^T      (A operands: tile rows)
//   P  = exp2(S c2 - lse2), dS = P * (dP - delta)
//   dV^T += dO^T . P,  dK^T += Q^T . dS   (A operands: transposed reads of
//                                          the same tiles)
// The 8 waves' partial dK^T, dV^T are folded through LDS at the end of the
// item by three halving exchanges, after which every wave stores one eighth.
// ---------------------------------------------------------------------------


// (m & a) | (~m & b), per 32-bit element
__device__ __forceinline__ float blend1(uint32_t m, float a, float b) {
  return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}
__device__ __forceinline__ float4 blend4(uint32_t m, float4 a, float4 b) {
  return make_float4(blend1(m, a.x, b.x), blend1(m, a.y, b.y), blend1(m, a.z, b.z),
                     blend1(m, a.w, b.w));
}

// One halving exchange of the dkdv fold.  Each of the NW waves holds N float4
// groups per lane in f[0, N); the wave with bit `bit` clear keeps the lower
// half, its partner (wave ^ bit) the upper half.  A wave writes the half it
// gives away to its own slot of `xch` (N/2 groups x 64 lanes) and, after a
// barrier, adds the partner's slot into the half it keeps, which it moves to
// f[0, N/2).  `pre_barrier`: wait first for every wave to be done with the
// LDS this level overwrites.
template <int N>
__device__ __forceinline__ void fold_level(const float4 (&f)[N], float4 (&out)[N / 2],
                                           float4* xch, int wave, int bit, int lane,
                                           bool pre_barrier) {
  constexpr int H = N / 2;
  if (pre_barrier) __syncthreads();
  // the halves are chosen with bit masks rather than a select, which the
  // compiler may turn into a run-time index that keeps f out of registers
  const uint32_t m = (wave & bit) ? 0xffffffffu : 0u;  // 1s: keep the upper half
  float4* mine = xch + (size_t)wave * H * 64 + lane;
#pragma unroll
  for (int i = 0; i < H; ++i) mine[i * 64] = blend4(m, f[i], f[H + i]);
  __syncthreads();
  const float4* theirs = xch + (size_t)(wave ^ bit) * H * 64 + lane;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float4 t = theirs[i * 64];
    const float4 k = blend4(m, f[H + i], f[i]);
    out[i] = make_float4(k.x + t.x, k.y + t.y, k.z + t.z, k.w + t.w);
  }
}

// One dkdv item: a 32-key tile, pairs [pbeg, pend) dealt to the 8 waves,
// fold, then the rows.
//   HIST = false: local key tile kt of the segment; pair pi = (query tile
//     kt + pi/G, head pi%G), causal; writes the final bf16 rows (plus, for the
//     exact gradient, the fp32 sums later segments left in a.hdk / a.hdv) or
//     (partial) the raw fp32 sums in slot pp.
//   HIST = true (exact gradient): the tile of history rows kbase ..
//     kbase+kvalid-1 of a block selected by the query blocks jlist[0..]; pair
//     pi = (jlist[pi / (G nq32)], then head and 32-query tile), every key
//     visible; adds its dK (scaled) and dV into a.hdk / a.hdv.
template <int D, bool HIST = false>
__device__ __forceinline__ void dkdv_item(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, float* __restrict__ pp,
    const BwdArgs& a, unsigned char* s_raw, int b, int g, int kt, int pbeg, int pend,
    bool partial, const int* jlist = nullptr, int kbase = 0, int kvalid = 0) {
  constexpr int TQ = 32;                 // queries per tile
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE_B = TQ * 2 * D;     // bytes of one row-major tile
  constexpr int SLICE_B = 2 * TILE_B + 256;  // Q tile, dO tile, lse + delta
  constexpr int NW = 8;
  const int t0 = a.seg * a.L;
  const int tend = t0 + a.L;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63, lq = lane & 31, hi = lane >> 5;
  unsigned char* s_k = s_raw;
  unsigned char* s_v = s_raw + TILE_B;
  unsigned char* s_q = s_raw + 2 * TILE_B + wave * SLICE_B;
  unsigned char* s_do = s_q + TILE_B;
  float* s_ld = reinterpret_cast<float*>(s_do + TILE_B);  // [0,32) lse, [32,64) delta
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;  // dK / dV rows (tokens)
  // K and V rows of this key tile, shared by the 8 waves (lane (key lq, hi)
  // reads K[key][16kk + 8hi .. +7]); the barrier also retires the previous
  // item's reads of the fold buffer that overlaps these tiles
  const int kfirst = HIST ? kbase : t0 + kt * 32;
  const int nkey = HIST ? kvalid : min(32, tend - kfirst);  // key rows that exist
  const int tk = kfirst + lq;
  const bool key_ok = lq < nkey;
  // the tile's first row in the K / V storage (its token in full-sequence
  // storage)
  const size_t kin = (size_t)(b * a.Hkv + g) * a.Skv * D + (size_t)(kfirst - t0 + a.kv_t0) * D;
  __syncthreads();
  if (wave == 0) dma_rows<D>(k + kin, 32, nkey, s_k, lane);
  if (wave == 1) dma_rows<D>(v + kin, 32, nkey, s_v, lane);
  drain_vmem_loads();
  __syncthreads();

  floatx16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkacc[db] = floatx16{}; dvacc[db] = floatx16{}; }
  FragOffsets<D> fo;
  fo.init(lane);

  for (int pi = pbeg + wave; pi < pend; pi += NW) {
    int h, tq0, nvalid;
    if constexpr (HIST) {
      const int per_j = a.G * a.nq32;
      const int jj = jlist[pi / per_j], rem = pi % per_j;
      const int qs = rem / a.G;
      h = g * a.G + rem % a.G;
      tq0 = t0 + jj * a.Bq + qs * TQ;
      nvalid = min(TQ, a.Bq - qs * TQ);
    } else {
      h = g * a.G + pi % a.G;
      tq0 = t0 + (kt + pi / a.G) * TQ;
      nvalid = min(TQ, tend - tq0);
    }
    const size_t hrow = (size_t)(b * a.Hq + h) * a.S;
    // stage the pair: tiles by direct loads, lse / delta one dword per lane
    dma_rows<D>(q + (hrow + tq0) * D, TQ, nvalid, s_q, lane);
    dma_rows<D>(dO + (hrow + tq0) * D, TQ, nvalid, s_do, lane);
    {
      const int tl = tq0 + min(lq, nvalid - 1);
      const float* src_ = hi == 0 ? lse + hrow + tl
                                  : delta + (size_t)(b * a.Hq + h) * a.L + (tl - t0);
      __builtin_amdgcn_global_load_lds((const void*)src_, to_lds(s_ld), 4, 0, 0);
    }
    drain_vmem_loads();
    wave_lds_sync();

    floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      sacc = mfma32(fo.row(s_q, 0, kk), fo.row(s_k, 0, kk), sacc);
      pacc = mfma32(fo.row(s_do, 0, kk), fo.row(s_v, 0, kk), pacc);
    }
    // the fragments of the next MFMA are requested before the current one
    // issues (two reads ahead), so LDS latency overlaps the matrix work
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int u = 0; u < 2 * NKK - 2; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    // C layout: lane = key lq, item r = query row 8(r/4)+4hi+(r%4) of the tile
    const bool need_mask = HIST ? (nvalid < TQ || nkey < 32)
                                : ((tq0 < kfirst + 31) || (nvalid < TQ) || (nkey < 32));
    float pv[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 l4 = *reinterpret_cast<const float4*>(&s_ld[8 * r4 + 4 * hi]);
      const float4 d4 = *reinterpret_cast<const float4*>(&s_ld[32 + 8 * r4 + 4 * hi]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv_[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * r4 + e;
        float p = fast_exp2(fmaf(sacc[r], a.c2, -lv[e] * kLog2e));
        if (need_mask) {
          const int row = 8 * r4 + 4 * hi + e;
          p = (key_ok && row < nvalid && (HIST || tk <= tq0 + row)) ? p : 0.f;
        }
        pv[r] = p;
        sacc[r] = p * (pacc[r] - dv_[e]);  // dS
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r0 = 8 * ks;
      const bf16x8 pb = to_bf16x8(pv[r0], pv[r0 + 1], pv[r0 + 2], pv[r0 + 3], pv[r0 + 4],
                                  pv[r0 + 5], pv[r0 + 6], pv[r0 + 7]);
      const bf16x8 sb = to_bf16x8(sacc[r0], sacc[r0 + 1], sacc[r0 + 2], sacc[r0 + 3],
                                  sacc[r0 + 4], sacc[r0 + 5], sacc[r0 + 6], sacc[r0 + 7]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvacc[db] = mfma32(fo.tr(s_do, 16 * ks, db), pb, dvacc[db]);
        dkacc[db] = mfma32(fo.tr(s_q, 16 * ks, db), sb, dkacc[db]);
      }
    }
    wave_lds_sync();  // this slice's reads are done before the next pair's loads land
  }

  // fold the 8 waves' partial sums by halving exchanges through LDS: at each
  // of three levels a wave sends the half of its list of float4 groups that
  // its partner (wave ^ 4, ^ 2, ^ 1) keeps and adds the partner's copy of the
  // half it keeps, so that wave w ends with groups [w NF/8, (w+1) NF/8) fully
  // summed.  Group f = (tensor, db, r4) holds items 4 r4 .. 4 r4 + 3 of
  // (tensor ? dV^T : dK^T)[db].  The first barrier also retires every wave's
  // reads of the K/V tiles and slices.
  constexpr int NF = 2 * NDB * 4;
  float4 f4[NF];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f4[db * 4 + r4] = make_float4(dkacc[db][4 * r4], dkacc[db][4 * r4 + 1],
                                    dkacc[db][4 * r4 + 2], dkacc[db][4 * r4 + 3]);
      f4[(NDB + db) * 4 + r4] = make_float4(dvacc[db][4 * r4], dvacc[db][4 * r4 + 1],
                                            dvacc[db][4 * r4 + 2], dvacc[db][4 * r4 + 3]);
    }
  float4* xch = reinterpret_cast<float4*>(s_raw);
  static_assert(NW == 8, "three halving levels");
  float4 f2[NF / 2], f3[NF / 4], f5[NF / 8];
  fold_level<NF>(f4, f2, xch, wave, 4, lane, true);
  fold_level<NF / 2>(f2, f3, xch, wave, 2, lane, true);
  // this level's slots lie beyond the previous level's: no barrier first
  fold_level<NF / 4>(f3, f5, xch + NW * (NF / 4) * 64, wave, 1, lane, false);

  // wave w stores groups f = w NF/8 + i
#pragma unroll
  for (int i = 0; i < NF / 8; ++i) {
    const int f = wave * (NF / 8) + i;
    const int tensor = f / (4 * NDB), db = (f / 4) % NDB, r4 = f % 4;
    const int d = 32 * db + 8 * r4 + 4 * hi;
    const float4 x = f5[i];
    if constexpr (HIST) {
      // exact gradient: this segment's part of the history rows' gradient
      if (key_ok) {
        float* dst = (tensor ? a.hdv : a.hdk) + kv_base + (size_t)tk * D + d;
        const float sc = tensor ? 1.f : a.scale;
        float4 y = *reinterpret_cast<float4*>(dst);
        y.x += x.x * sc; y.y += x.y * sc; y.z += x.z * sc; y.w += x.w * sc;
        *reinterpret_cast<float4*>(dst) = y;
      }
    } else if (partial) {
      // raw fp32 rows [dK^T keys 0..31 | dV^T keys 0..31] x D, added by the
      // dq kernel that follows in the same backward call
      *reinterpret_cast<float4*>(pp + (size_t)(32 * tensor + lq) * D + d) = x;
    } else if (key_ok) {
      const float sc = tensor ? 1.f : a.scale;
      float4 hx = make_float4(0.f, 0.f, 0.f, 0.f);
      if (a.hdk != nullptr)  // exact gradient: what later segments added
        hx = *reinterpret_cast<const float4*>((tensor ? a.hdv : a.hdk) + kv_base +
                                              (size_t)tk * D + d);
      const bf16x4 o4 = {(__bf16)(x.x * sc + hx.x), (__bf16)(x.y * sc + hx.y),
                         (__bf16)(x.z * sc + hx.z), (__bf16)(x.w * sc + hx.w)};
      *reinterpret_cast<bf16x4*>((tensor ? dv : dk) + kv_base + (size_t)tk * D + d) = o4;
    }
  }
}

template <int D>
__global__ __launch_bounds__(512) void dkdv_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, float* __restrict__ part_ws, BwdArgs a) {
  constexpr int TQ = 32;
  constexpr int NDB = D / 32;
  constexpr int TILE_B = TQ * 2 * D;
  constexpr int SLICE_B = 2 * TILE_B + 256;
  constexpr int NW = 8;
  constexpr int FOLD_B = NW * (2 * NDB * 4 / 2) * 64 * 16;  // first fold level's slots
  constexpr int STAGE_B = 2 * TILE_B + NW * SLICE_B;  // K, V tiles + wave slices
  constexpr int LDS_BYTES = STAGE_B > FOLD_B ? STAGE_B : FOLD_B;
  __shared__ __attribute__((aligned(1024))) unsigned char s_raw[LDS_BYTES];

  const int nkt = (a.L + 31) / 32;
  const int nbk = nkt + (nkt & 1);  // blocks per (b, g)
  const int nph = (nkt + 1) / 2;    // mirror pairs (partial-sum slots)
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int n = w % nbk;
  const int g = (w / nbk) % a.Hkv;
  const int b = w / (nbk * a.Hkv);
  // block 2p: pairs [0, split) of tile p; block 2p+1: the rest of tile p,
  // then the mirror tile (scalars only, nothing indexed at run time)
  const int p = n >> 1, part = n & 1;
  const int wh = a.G * (nkt - p);
  const int wl = dkdv_mirror_pairs(p, nkt, a.G);
  const int split = dkdv_split(wh, wl);
  const bool tile_split = split < wh;
  const bool rest_first = part == 1 && tile_split;
  const int kt1 = (part == 0 || tile_split) ? p : nkt - 1 - p;
  const int b1 = rest_first ? split : 0;
  const int e1 = part == 0 ? split : (tile_split ? wh : wl);
  const bool has2 = rest_first && wl > 0;
  float* pp = part_ws + ((size_t)((b * a.Hkv + g) * nph + p) * 2 + part) * 64 * D;
  if (e1 > b1)
    dkdv_item<D>(q, k, v, lse, dO, delta, dk, dv, pp, a, s_raw, b, g, kt1, b1, e1,
                 kt1 == p && tile_split);
  if (has2)
    dkdv_item<D>(q, k, v, lse, dO, delta, dk, dv, pp, a, s_raw, b, g, nkt - 1 - p, 0, wl, false);
}



// ---------------------------------------------------------------------------
// a8, bf16 MFMA, whole segmented pass: dk/dv of the local keys of segments
// a.seg .. a.seg+a.nseg-1 in one launch.  A block of 4 waves takes two key
// blocks of 128 consecutive keys of one (segment, b, g), kb and its mirror
// nkb-1-kb, one after the other; for each, wave w owns keys k0+32w .. +31,
// holds their K rows in registers (B operand of S = Q.K^T), their V rows in
// LDS (B operand of dP = dO.V^T) and their dK^T, dV^T accumulators.  The
// block walks the (32-query tile, head) pairs that can see the key block --
// query tiles from its first key on, every head of the group -- and copies
// each pair's Q and dO tiles (with lse and delta) into LDS once for its 4
// waves, double-buffered so that the next pair's copies land while the
// current one is computed.  Per wave and pair, with the products of
// dkdv_item:
//   S = Q.K^T, dP = dO.V^T,  P = exp2(S c2 - lse2), dS = P (dP - delta)
//   dV^T += dO^T.P,  dK^T += Q^T.dS      (transposed reads of the Q, dO tiles)
// Each key has one owner, so its dK, dV rows are written directly (plus,
// for the exact gradient, the fp32 sums a.hdk / a.hdv that later segments'
// queries left in those rows).
//
// Work order: key block kb sees nqt - 4kb query tiles (32-row tiles, L/32
// of them), so the pair kb, nkb-1-kb gives every block the same work.  The
// blocks of one (segment, b, g) are consecutive, so they run together on
// one XCD, and they read the same Q/dO tiles at the same time: the first
// key block walks its query tiles from the last down (tile nqt-1-t at step
// t in every block), the second from its first tile up, which every block
// reaches at the same step (tile t - nqt/8 at step t for L = 1024).  Each
// tile is thus read from memory about once per direction, and the L2
// serves the other blocks.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void dkdv_pass_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, BwdArgs a) {
  constexpr int TQ = 32;                 // queries per tile
  constexpr int KB = 128;                // keys per block
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE_B = TQ * 2 * D;     // bytes of one 32-row tile
  constexpr int STAGE_B = 2 * TILE_B + 512;  // Q tile, dO tile, lse (64), delta (64)
  constexpr int CPR = (2 * D) / 16;
  constexpr int RPI = 64 / CPR;          // rows per 1 KB copy instruction
  __shared__ __attribute__((aligned(1024))) unsigned char s_v[KB * 2 * D];
  __shared__ __attribute__((aligned(1024))) unsigned char s_stage[2][STAGE_B];

  const int nkb = (a.L + KB - 1) / KB;
  const int nbpg = (nkb + 1) / 2;  // blocks per (segment, b, g)
  int w = xcd_remap(blockIdx.x, gridDim.x);
  const int pr = w % nbpg;
  w /= nbpg;
  const int sg = a.nseg - 1 - w % a.nseg;
  w /= a.nseg;
  const int g = w % a.Hkv;
  const int b = w / a.Hkv;
  const int seg = a.seg + sg;
  const int t0 = seg * a.L, tend = t0 + a.L;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane_id = tid & 63;
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;
  const float* dlt = delta + (size_t)sg * a.dchunk;
  const int nqt = (a.L + TQ - 1) / TQ;
  FragOffsets<D> fo;
  fo.init(lane_id);
  const unsigned char* vt = s_v + wave * 32 * (2 * D);

  // key block pr, its query tiles from the last down, then key block
  // nkb-1-pr, its query tiles from the first up (nothing more for the middle
  // block of an odd nkb)
  const int nphase = nkb - 1 - pr != pr ? 2 : 1;
  for (int ph = 0; ph < nphase; ++ph) {
    // the lane index, opaque to the compiler, so that the offsets derived
    // from it are recomputed per key block rather than held through the
    // pair loop
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int lq = lane & 31, hi = lane >> 5;
    const int kb = ph == 0 ? pr : nkb - 1 - pr;
    const bool down = ph == 0;
    const int k0 = t0 + kb * KB;
    // keys of this wave; rows past the segment end read the last row (masked)
    const int kfirst = k0 + 32 * wave;
    const int nkey = max(0, min(32, tend - kfirst));
    const int tk = kfirst + lq;
    const bool key_ok = lq < nkey;
    const int nkey_blk = min(KB, tend - k0);
    if (ph > 0) __syncthreads();  // every wave is done with the first key block's tiles
    // V rows of the block's keys into LDS (4 waves x 8 instructions)
    {
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(v + kv_base + (size_t)k0 * D, (uint32_t)nkey_blk * (2 * D));
#pragma unroll
      for (int n = 0; n < KB / RPI / 4; ++n) {
        const int i = wave + 4 * n;
        const int row = i * RPI + lane / CPR;
        const int c = (lane % CPR) ^ swz<D>(row);
        const int rr = row < nkey_blk ? row : nkey_blk - 1;
        buffer_to_lds16(r, (uint32_t)rr * (2 * D) + c * 16, s_v + i * 1024);
      }
    }
    // K rows of this wave's keys as B operands: lane (key lq, hi) holds
    // K[key][16kk + 8hi .. +7]
    bf16x8 kreg[NKK];
    {
      const int krow = key_ok ? tk : (nkey > 0 ? kfirst : tend - 1);
      const __bf16* kp = k + kv_base + (size_t)krow * D + 8 * hi;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) kreg[kk] = *reinterpret_cast<const bf16x8*>(kp + 16 * kk);
    }

    const int qt0 = (kb * KB) / TQ;        // first query tile that sees any key
    const int npairs = (nqt - qt0) * a.G;
    auto tile_of = [&](int pi) { return down ? nqt - 1 - pi / a.G : qt0 + pi / a.G; };
    // copies of pair pi's tiles (every wave a quarter of Q and dO; waves 0 / 1
    // the lse / delta of its 32 queries) into stage buffer `st`
    auto stage_pair = [&](int pi, int st) __attribute__((always_inline)) {
      const bool ok = pi < npairs;
      const int pc = ok ? pi : 0;
      const int qt = tile_of(pc), h = g * a.G + pc % a.G;
      const int tq0 = t0 + qt * TQ;
      const int nval = min(TQ, tend - tq0);
      const size_t hrow = (size_t)(b * a.Hq + h) * a.S;
      const uint32_t nb = ok ? (uint32_t)nval * (2 * D) : 0u;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + (hrow + tq0) * D, nb);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(dO + (hrow + tq0) * D, nb);
      unsigned char* sq = s_stage[st];
      unsigned char* sd = sq + TILE_B;
#pragma unroll
      for (int n = 0; n < TQ / RPI / 4; ++n) {
        const int i = wave + 4 * n;
        const int row = i * RPI + lane / CPR;
        const int c = (lane % CPR) ^ swz<D>(row);
        const int rr = row < nval ? row : nval - 1;
        buffer_to_lds16(rq, (uint32_t)rr * (2 * D) + c * 16, sq + i * 1024);
        buffer_to_lds16(rd, (uint32_t)rr * (2 * D) + c * 16, sd + i * 1024);
      }
      if (wave < 2) {
        const float* base = wave == 0 ? lse + hrow + tq0
                                      : dlt + (size_t)(b * a.Hq + h) * a.L + (tq0 - t0);
        const __amdgpu_buffer_rsrc_t rl = make_rsrc(base, ok ? (uint32_t)nval * 4u : 0u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, to_lds(sq + 2 * TILE_B + wave * 256), 4,
                                                 (int)((lane & 31) * 4), 0, 0, 0);
      }
    };

    floatx16 dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) { dkacc[db] = floatx16{}; dvacc[db] = floatx16{}; }

    stage_pair(0, 0);
    drain_vmem_loads();
    __syncthreads();

    for (int pi = 0; pi < npairs; ++pi) {
      stage_pair(pi + 1, (pi + 1) & 1);
      const int tq0 = t0 + tile_of(pi) * TQ;
      const int nval = min(TQ, tend - tq0);
      // a wave whose keys all come after the tile's queries has nothing to do
      if (nkey > 0 && tq0 + TQ - 1 >= kfirst) {
        const unsigned char* sq = s_stage[pi & 1];
        const unsigned char* sd = sq + TILE_B;
        const float* sl = reinterpret_cast<const float*>(sq + 2 * TILE_B);
        floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sacc = mfma32(fo.row(sq, 0, kk), kreg[kk], sacc);
          pacc = mfma32(fo.row(sd, 0, kk), fo.row(vt, 0, kk), pacc);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int u = 0; u < 2 * NKK - 2; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        // C layout: lane = key lq, item r = query row 8(r/4)+4hi+(r%4) of the tile
        const bool need_mask = (tq0 < kfirst + 31) || (nval < TQ) || (nkey < 32);
        float pv[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 l4 = *reinterpret_cast<const float4*>(&sl[8 * r4 + 4 * hi]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pv[4 * r4 + e] = fast_exp2(fmaf(sacc[4 * r4 + e], a.c2, -lv[e] * kLog2e));
        }
        if (need_mask) {
          // kept a branch (a fence with side effects): only diagonal and
          // ragged pairs need it
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * hi + (r & 3);
            pv[r] = (key_ok && row < nval && tk <= tq0 + row) ? pv[r] : 0.f;
          }
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {  // dS
          const float4 d4 = *reinterpret_cast<const float4*>(&sl[64 + 8 * r4 + 4 * hi]);
          const float dv_[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[4 * r4 + e] = pv[4 * r4 + e] * (pacc[4 * r4 + e] - dv_[e]);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 8 * ks;
          const bf16x8 pb = to_bf16x8(pv[r0], pv[r0 + 1], pv[r0 + 2], pv[r0 + 3], pv[r0 + 4],
                                      pv[r0 + 5], pv[r0 + 6], pv[r0 + 7]);
          const bf16x8 sb = to_bf16x8(sacc[r0], sacc[r0 + 1], sacc[r0 + 2], sacc[r0 + 3],
                                      sacc[r0 + 4], sacc[r0 + 5], sacc[r0 + 6], sacc[r0 + 7]);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dvacc[db] = mfma32(fo.tr(sd, 16 * ks, db), pb, dvacc[db]);
            dkacc[db] = mfma32(fo.tr(sq, 16 * ks, db), sb, dkacc[db]);
          }
        }
      }
      drain_vmem_loads();  // the next pair's tiles have landed
      __syncthreads();
    }

    if (key_ok) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = 32 * db + 8 * r4 + 4 * hi;
          const size_t off = kv_base + (size_t)tk * D + d;
          float4 hk = make_float4(0.f, 0.f, 0.f, 0.f), hv = hk;
          if (a.hdk != nullptr) {
            hk = *reinterpret_cast<const float4*>(a.hdk + off);
            hv = *reinterpret_cast<const float4*>(a.hdv + off);
          }
          const bf16x4 ko = {(__bf16)(dkacc[db][4 * r4] * a.scale + hk.x),
                             (__bf16)(dkacc[db][4 * r4 + 1] * a.scale + hk.y),
                             (__bf16)(dkacc[db][4 * r4 + 2] * a.scale + hk.z),
                             (__bf16)(dkacc[db][4 * r4 + 3] * a.scale + hk.w)};
          const bf16x4 vo = {(__bf16)(dvacc[db][4 * r4] + hv.x),
                             (__bf16)(dvacc[db][4 * r4 + 1] + hv.y),
                             (__bf16)(dvacc[db][4 * r4 + 2] + hv.z),
                             (__bf16)(dvacc[db][4 * r4 + 3] + hv.w)};
          *reinterpret_cast<bf16x4*>(dk + off) = ko;
          *reinterpret_cast<bf16x4*>(dv + off) = vo;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Exact-gradient backward ([SeCO] 提案手法: the chunks are visited from the
// last one and the gradient is exact; here the history keys of a segment
// are not detached).  The segment's queries also give dK/dV to the history
// blocks they selected.  hist_blocks_kernel lists, per (sequence, KV head),
// every distinct selected block, ascending, with the mask of the query
// blocks that chose it (an LDS bit table per history block, filled by
// integer ORs, then compacted with ballots); dkdv_hist_kernel then walks (block,
// 32-key tile) items, each owned by one block of threads, which adds the
// tile's dK/dV into the fp32 sums a.hdk / a.hdv (no atomics: one owner per
// row, so the sums are deterministic).
// ---------------------------------------------------------------------------
struct HistEntry {
  int blk;
  int pad;
  unsigned long long jmask;  // bit j: query block j of the segment chose blk
};


// One block of threads per (sequence, KV head) and segment a.seg +
// blockIdx.y; segment a.seg + y writes its list and counts at list +
// y * list_stride and counts + y * count_stride (whole-pass form: every
// segment's list in one launch).
__global__ __launch_bounds__(256) void hist_blocks_kernel(const int32_t* __restrict__ sel,
                                                          HistEntry* __restrict__ list,
                                                          int* __restrict__ counts, BwdArgs a,
                                                          int maxd, size_t list_stride,
                                                          int count_stride) {
  __shared__ unsigned long long s_mask[kMaxCandidates];  // per history block
  __shared__ int s_wtot[4];
  const int bg = blockIdx.x;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int seg = a.seg + (int)blockIdx.y;
  list += blockIdx.y * list_stride;
  counts += blockIdx.y * count_stride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = seg * a.L / a.Bh;
  const int n_ent = a.nqb * a.K;
  const int32_t* rows = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)seg * a.nqb) * a.K;
  for (int i = tid; i < nb; i += 256) s_mask[i] = 0ull;
  __syncthreads();
  // bit j of block x's mask: query block j chose x (integer OR: the result
  // does not depend on the order of the updates)
  for (int e = tid; e < n_ent; e += 256) {
    const int x = rows[e];
    if (x >= 0 && x < nb) atomicOr(&s_mask[x], 1ull << (e / a.K));
  }
  __syncthreads();
  // the chosen blocks in ascending order
  int count = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int base = 0; base < nb; base += 256) {
    const int i = base + tid;
    const unsigned long long m = i < nb ? s_mask[i] : 0ull;
    const unsigned long long bal = __ballot(m != 0ull);
    if (lane == 0) s_wtot[wave] = __popcll(bal);
    __syncthreads();
    int off = count;
    for (int w = 0; w < wave; ++w) off += s_wtot[w];
    if (m != 0ull) {
      HistEntry* out = list + (size_t)bg * maxd + off + __popcll(bal & below);
      out->blk = i;
      out->pad = 0;
      out->jmask = m;
    }
    count += s_wtot[0] + s_wtot[1] + s_wtot[2] + s_wtot[3];
    __syncthreads();
  }
  if (tid == 0) counts[bg] = count;
}

template <int D>
__global__ __launch_bounds__(512) void dkdv_hist_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    const HistEntry* __restrict__ list, const int* __restrict__ counts, BwdArgs a, int maxd,
    int ntpb) {
  constexpr int TQ = 32;
  constexpr int NDB = D / 32;
  constexpr int TILE_B = TQ * 2 * D;
  constexpr int SLICE_B = 2 * TILE_B + 256;
  constexpr int NW = 8;
  constexpr int STAGE_B = 2 * TILE_B + NW * SLICE_B;
  constexpr int FOLD_B = NW * (2 * NDB * 4 / 2) * 64 * 16;
  constexpr int LDS_BYTES = STAGE_B > FOLD_B ? STAGE_B : FOLD_B;
  __shared__ __attribute__((aligned(1024))) unsigned char s_raw[LDS_BYTES];
  __shared__ int s_j[64];
  __shared__ int s_nj;
  const int nbg = a.B * a.Hkv;
  const int total = maxd * ntpb * nbg;
  // items t = (entry idx, key tile kt, bg) with bg fastest, so that the live
  // entries (idx < count) come first and are dealt evenly over the grid
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int bg = t % nbg, rest = t / nbg;
    const int kt = rest % ntpb, idx = rest / ntpb;
    if (idx >= counts[bg]) continue;  // uniform over the block
    const HistEntry ent = list[(size_t)bg * maxd + idx];
    __syncthreads();  // the previous item's reads of s_j are done
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const bool bit = lane < a.nqb && ((ent.jmask >> lane) & 1ull);
      const unsigned long long m = __ballot(bit);
      if (bit) s_j[__popcll(m & ((1ull << lane) - 1ull))] = lane;
      if (lane == 0) s_nj = __popcll(m);
    }
    __syncthreads();
    const int pairs = s_nj * a.G * a.nq32;
    dkdv_item<D, true>(q, k, v, lse, dO, delta, nullptr, nullptr, nullptr, a, s_raw,
                       bg / a.Hkv, bg % a.Hkv, kt, 0, pairs, false, s_j,
                       ent.blk * a.Bh + 32 * kt, min(32, a.Bh - 32 * kt));
  }
}

// Clears n floats (n a multiple of 4, 16-byte aligned): a plain store kernel,
// so that it may sit in a captured graph.
__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// float32 kernels (reference-precision path, plain VALU).
// dq: one query per lane, key tiles of 32 rows in LDS (same key order as the
// forward).  dk/dv: one local key per lane, query tiles of 32 rows of each
// head of the group in LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dO,
    const float* __restrict__ delta, const int32_t* __restrict__ sel,
    float* __restrict__ dq, BwdArgs a) {
  constexpr int TKF = 32;
  __shared__ float s_k[TKF][D];
  __shared__ float s_v[TKF][D];
  __shared__ int s_hlist[kMaxTopK];
  __shared__ int s_hcount;

  const int nch = (a.Bq + 63) / 64;
  int w = blockIdx.x;
  const int ch = w % nch; w /= nch;
  const int j = w % a.nqb; w /= a.nqb;
  const int h = w % a.Hq;
  const int b = w / a.Hq;
  const int g = h / a.G;
  const int t0 = a.seg * a.L;
  const int nb = t0 / a.Bh;
  const int lane = threadIdx.x;
  const int qoff = ch * 64 + lane;
  const bool row_ok = qoff < a.Bq;
  const int tq = t0 + j * a.Bq + min(qoff, a.Bq - 1);
  const int qmax = t0 + j * a.Bq + min(ch * 64 + 63, a.Bq - 1);

  const int32_t* srow = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)a.seg * a.nqb + j) * a.K;
  const int nsel = compact_selection(srow, a.K, nb, s_hlist, &s_hcount);
  const int nh = nsel * a.Bh;
  const int nkeys = nh + (qmax - t0 + 1);

  const size_t qrow = (size_t)(b * a.Hq + h) * a.S + tq;
  float qr[D], dor[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { qr[d] = q[qrow * D + d]; dor[d] = dO[qrow * D + d]; acc[d] = 0.f; }
  const float lq = lse[qrow];
  const float dl = delta[(size_t)(b * a.Hq + h) * a.L + (tq - t0)];
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;

  for (int base = 0; base < nkeys; base += TKF) {
    for (int e = lane; e < TKF * D; e += 64) {
      const int r = e / D, d = e % D;
      const int slot = base + r;
      int tok = -1;
      if (slot < nh) tok = s_hlist[slot / a.Bh] * a.Bh + slot % a.Bh;
      else if (slot < nkeys) tok = t0 + (slot - nh);
      s_k[r][d] = tok >= 0 ? k[kv_base + (size_t)tok * D + d] : 0.f;
      s_v[r][d] = tok >= 0 ? v[kv_base + (size_t)tok * D + d] : 0.f;
    }
    __syncthreads();
    const int n = min(TKF, nkeys - base);
    for (int r = 0; r < n; ++r) {
      const int slot = base + r;
      if (slot >= nh && t0 + (slot - nh) > tq) continue;
      float z = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) { z += qr[d] * s_k[r][d]; dp += dor[d] * s_v[r][d]; }
      const float p = expf(z * a.scale - lq);
      const float ds = p * (dp - dl);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] += ds * s_k[r][d];
    }
    __syncthreads();
  }
  if (row_ok) {
#pragma unroll
    for (int d = 0; d < D; ++d) dq[qrow * D + d] = acc[d] * a.scale;
  }
}

template <int D>
__global__ __launch_bounds__(64) void dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dO,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv,
    BwdArgs a) {
  constexpr int TQF = 32;
  __shared__ float s_q[TQF][D];
  __shared__ float s_do[TQF][D];
  __shared__ float s_l[TQF], s_dl[TQF];

  const int nch = (a.L + 63) / 64;
  int w = blockIdx.x;
  const int ch = w % nch; w /= nch;
  const int g = w % a.Hkv;
  const int b = w / a.Hkv;
  const int t0 = a.seg * a.L, tend = t0 + a.L;
  const int lane = threadIdx.x;
  const int tk = t0 + ch * 64 + lane;
  const bool key_ok = tk < tend;
  const int tkc = key_ok ? tk : tend - 1;
  const int kmin = t0 + ch * 64;
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;

  float kr[D], vr[D], dka[D], dva[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kr[d] = k[kv_base + (size_t)tkc * D + d];
    vr[d] = v[kv_base + (size_t)tkc * D + d];
    dka[d] = 0.f;
    dva[d] = 0.f;
  }
  for (int hh = 0; hh < a.G; ++hh) {
    const int h = g * a.G + hh;
    const size_t hrow = (size_t)(b * a.Hq + h) * a.S;
    for (int base = kmin; base < tend; base += TQF) {
      for (int e = lane; e < TQF * D; e += 64) {
        const int r = e / D, d = e % D;
        const int t = base + r;
        s_q[r][d] = t < tend ? q[(hrow + t) * D + d] : 0.f;
        s_do[r][d] = t < tend ? dO[(hrow + t) * D + d] : 0.f;
      }
      for (int r = lane; r < TQF; r += 64) {
        const int t = base + r;
        s_l[r] = t < tend ? lse[hrow + t] : 0.f;
        s_dl[r] = t < tend ? delta[(size_t)(b * a.Hq + h) * a.L + (t - t0)] : 0.f;
      }
      __syncthreads();
      const int n = min(TQF, tend - base);
      for (int r = 0; r < n; ++r) {
        if (base + r < tk) continue;  // query before this key: no contribution
        float z = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) { z += s_q[r][d] * kr[d]; dp += s_do[r][d] * vr[d]; }
        const float p = expf(z * a.scale - s_l[r]);
        const float ds = p * (dp - s_dl[r]);
#pragma unroll
        for (int d = 0; d < D; ++d) { dka[d] += ds * s_q[r][d]; dva[d] += p * s_do[r][d]; }
      }
      __syncthreads();
    }
  }
  if (key_ok) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      dk[kv_base + (size_t)tk * D + d] = dka[d] * a.scale;
      dv[kv_base + (size_t)tk * D + d] = dva[d];
    }
  }
}

BwdArgs make_args(const Prob& p, int seg) {
  BwdArgs a;
  a.B = p.B;
  a.S = p.S; a.L = p.L; a.Bh = p.Bh; a.Bq = p.Bq; a.K = p.K; a.Hq = p.Hq; a.Hkv = p.Hkv;
  a.G = p.G; a.nqb = p.nqb; a.nqb_all = p.nqb_all; a.seg = seg;
  a.nq32 = (p.Bq + 31) / 32;
  a.wpu = (p.G * a.nq32 + 3) / 4;
  a.c2 = p.scale * kLog2e;
  a.scale = p.scale;
  a.hdk = a.hdv = nullptr;
  a.nseg = 1;
  a.dchunk = 0;
  a.Skv = p.kv_rows;
  a.kv_t0 = p.kv_local >= 0 ? p.kv_local : seg * p.L;
  return a;
}

// Backward workspace: delta [B, Hq, L] fp32, then the dK/dV partial sums of
// the mirror-paired key tiles, [B, Hkv, nph, 2, 64, D] fp32.
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t dkdv_slots(const Prob& p) {
  const size_t nph = ((size_t)(p.L + 31) / 32 + 1) / 2;
  return (size_t)p.B * p.Hkv * nph;
}
size_t delta_bytes(const Prob& p) { return round256((size_t)p.B * p.Hq * p.L * sizeof(float)); }
size_t partial_bytes(const Prob& p) {
  return round256(dkdv_slots(p) * 2 * 64 * p.D * sizeof(float));
}
float* dkdv_partials(const Prob& p, float* delta) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(delta) + delta_bytes(p));
}
// exact backward: after the above, per (b, g) a count and up to maxd entries
int hist_max_entries(const Prob& p) {
  const int nb_max = (p.S - p.L) / p.Bh;
  const int n_ent = p.nqb * p.K;
  return nb_max < n_ent ? nb_max : n_ent;
}
size_t hist_list_bytes(const Prob& p) {
  return round256((size_t)p.B * p.Hkv * sizeof(int)) +
         round256((size_t)p.B * p.Hkv * (hist_max_entries(p) > 0 ? hist_max_entries(p) : 1) *
                  sizeof(HistEntry));
}

template <typename T, int D>
hipError_t delta_t(const Prob& p, const void* o, const void* dO, int seg, float* delta,
                   hipStream_t st) {
  constexpr int C = D / Vec16<T>::N;
  constexpr int RPB = 256 / C;
  const int nrows = p.B * p.Hq * p.L;
  HGA_LAUNCH(HGA_K_BWD_PRE, (delta_kernel<T, D>), dim3((nrows + RPB - 1) / RPB), dim3(256), 0, st,
                     (const T*)o, (const T*)dO, delta, p.S, p.L, seg * p.L, nrows);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_bf16(const Prob& p, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dO, const int32_t* sel,
                    int seg, void* dq, void* dk, void* dv, float* delta, hipStream_t st,
                    bool delta_ready, float* hdk, float* hdv, float* partials) {
  hipError_t e = delta_ready ? hipSuccess : delta_t<__bf16, D>(p, o, dO, seg, delta, st);
  if (e != hipSuccess) return e;
  BwdArgs a = make_args(p, seg);
  a.hdk = hdk;
  a.hdv = hdv;
  const int nkt = (p.L + 31) / 32;
  const int nph = (nkt + 1) / 2;
  float* part_ws = partials != nullptr ? partials : dkdv_partials(p, delta);
  {
    // dk/dv first: the dq kernel finishes the key tiles it left as partial sums
    const int nblocks = p.B * p.Hkv * (nkt + (nkt & 1));
    HGA_LAUNCH(HGA_K_BWD_DKDV, (dkdv_bf16_kernel<D>), dim3(nblocks), dim3(512), 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, lse,
                       (const __bf16*)dO, delta, (__bf16*)dk, (__bf16*)dv, part_ws, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int maxd = hist_max_entries(p);
  if (hdk != nullptr && seg > 0 && maxd > 0) {
    // exact gradient: this segment's contribution to its history blocks
    char* base = reinterpret_cast<char*>(part_ws) + partial_bytes(p);
    int* counts = reinterpret_cast<int*>(base);
    HistEntry* list =
        reinterpret_cast<HistEntry*>(base + round256((size_t)p.B * p.Hkv * sizeof(int)));
    HGA_LAUNCH(HGA_K_BWD_HIST, hist_blocks_kernel, dim3(p.B * p.Hkv), dim3(256), 0, st, sel, list,
               counts, a, maxd, (size_t)0, 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ntpb = (p.Bh + 31) / 32;
    HGA_LAUNCH(HGA_K_BWD_HIST, (dkdv_hist_kernel<D>), dim3(256), dim3(512), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, lse, (const __bf16*)dO, delta,
                       (const HistEntry*)list, (const int*)counts, a, maxd, ntpb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nblocks = p.B * p.Hkv * p.nqb * a.wpu;
    HGA_LAUNCH(HGA_K_BWD_DQ, (dq_bf16_kernel<D>), dim3(nblocks), dim3(512), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, lse, (const __bf16*)dO, delta, sel,
                       (__bf16*)dq, part_ws, (__bf16*)dk, (__bf16*)dv, nph, a);
    e = hipGetLastError();
  }
  return e;
}

// Backward of segments seg0 .. seg0+nseg-1 in two launches, dkdv then dq;
// each segment's delta rows at the given stride (bytes).
template <int D>
hipError_t bwd_pass_bf16(const Prob& p, const void* q, const void* k, const void* v,
                         const float* lse, const void* dO, const int32_t* sel, int seg0,
                         int nseg, void* dq, void* dk, void* dv, const float* delta,
                         size_t dstride, hipStream_t st, const float* hdk, const float* hdv) {
  BwdArgs a = make_args(p, seg0);
  a.nseg = nseg;
  a.dchunk = (int)(dstride / sizeof(float));
  a.hdk = const_cast<float*>(hdk);
  a.hdv = const_cast<float*>(hdv);
  {
    const int nkb = (p.L + 127) / 128;
    const int nblocks = p.B * p.Hkv * nseg * ((nkb + 1) / 2);
    HGA_LAUNCH(HGA_K_BWD_DKDV, (dkdv_pass_kernel<D>), dim3(nblocks), dim3(256), 0, st,
               (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, lse, (const __bf16*)dO,
               delta, (__bf16*)dk, (__bf16*)dv, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nblocks = p.B * p.Hkv * nseg * p.nqb * a.wpu;
  HGA_LAUNCH(HGA_K_BWD_DQ, (dq_pass_kernel<D>), dim3(nblocks), dim3(256), 0, st,
             (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, lse, (const __bf16*)dO, delta,
             sel, (__bf16*)dq, a);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_f32(const Prob& p, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dO, const int32_t* sel,
                   int seg, void* dq, void* dk, void* dv, float* delta, hipStream_t st) {
  hipError_t e = delta_t<float, D>(p, o, dO, seg, delta, st);
  if (e != hipSuccess) return e;
  BwdArgs a = make_args(p, seg);
  {
    const int nblocks = p.B * p.Hq * p.nqb * ((p.Bq + 63) / 64);
    HGA_LAUNCH(HGA_K_BWD_DQ, (dq_f32_kernel<D>), dim3(nblocks), dim3(64), 0, st, (const float*)q,
                       (const float*)k, (const float*)v, lse, (const float*)dO, delta, sel,
                       (float*)dq, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nblocks = p.B * p.Hkv * ((p.L + 63) / 64);
    HGA_LAUNCH(HGA_K_BWD_DKDV, (dkdv_f32_kernel<D>), dim3(nblocks), dim3(64), 0, st,
               (const float*)q,
                       (const float*)k, (const float*)v, lse, (const float*)dO, delta,
                       (float*)dk, (float*)dv, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

size_t bwd_workspace_bytes(const Prob& p) {
  return delta_bytes(p) + partial_bytes(p);
}

size_t bwd_delta_bytes(const Prob& p) { return delta_bytes(p); }

hipError_t launch_bwd_pass(const Prob& p, const void* q, const void* k, const void* v,
                           const float* lse, const void* dO, const int32_t* sel, int seg0,
                           int nseg, void* dq, void* dk, void* dv, const float* delta,
                           size_t dstride, hipStream_t st, const float* hist_dk,
                           const float* hist_dv) {
  if (p.dtype != HGA_BF16 || p.kv_rows != p.S) return hipErrorInvalidValue;
  return p.D == 64 ? bwd_pass_bf16<64>(p, q, k, v, lse, dO, sel, seg0, nseg, dq, dk, dv, delta,
                                       dstride, st, hist_dk, hist_dv)
                   : bwd_pass_bf16<128>(p, q, k, v, lse, dO, sel, seg0, nseg, dq, dk, dv, delta,
                                        dstride, st, hist_dk, hist_dv);
}

hipError_t launch_zero(float* p, size_t n, hipStream_t st) {
  const size_t n4 = n / 4;
  const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 4096);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, st, (float4*)p, n4);
  return hipGetLastError();
}



// Segment seg's list in the lists workspace (hist_lists_bytes): segments
// 1 .. S/L-1, each hist_list_bytes, counts first.
static void hist_list_of(const Prob& p, void* lists_ws, int seg, int** counts,
                         HistEntry** list) {
  char* base = reinterpret_cast<char*>(lists_ws) + (size_t)(seg - 1) * hist_list_bytes(p);
  *counts = reinterpret_cast<int*>(base);
  *list = reinterpret_cast<HistEntry*>(base + round256((size_t)p.B * p.Hkv * sizeof(int)));
}

size_t hist_lists_bytes(const Prob& p) {
  return (size_t)(p.S / p.L > 1 ? p.S / p.L - 1 : 1) * hist_list_bytes(p);
}

hipError_t launch_hist_lists(const Prob& p, const int32_t* sel, void* lists_ws,
                             hipStream_t st) {
  const int maxd = hist_max_entries(p);
  const int nseg = p.S / p.L;
  if (nseg <= 1 || maxd <= 0) return hipSuccess;
  BwdArgs a = make_args(p, 1);
  int* counts;
  HistEntry* list;
  hist_list_of(p, lists_ws, 1, &counts, &list);
  const size_t stride = hist_list_bytes(p);  // bytes; both strides below in elements
  HGA_LAUNCH(HGA_K_BWD_HIST, hist_blocks_kernel, dim3(p.B * p.Hkv, nseg - 1), dim3(256), 0, st,
             sel, list, counts, a, maxd, stride / sizeof(HistEntry),
             (int)(stride / sizeof(int)));
  return hipGetLastError();
}

hipError_t launch_hist_exact(const Prob& p, const void* q, const void* k, const void* v,
                             const float* lse, const void* dO, const int32_t* sel, int seg,
                             const float* delta_seg, float* hist_dk, float* hist_dv,
                             void* lists_ws, hipStream_t st) {
  (void)sel;
  if (p.dtype != HGA_BF16 || p.kv_rows != p.S) return hipErrorInvalidValue;
  const int maxd = hist_max_entries(p);
  if (seg <= 0 || maxd <= 0) return hipSuccess;
  BwdArgs a = make_args(p, seg);
  a.hdk = hist_dk;
  a.hdv = hist_dv;
  int* counts;
  HistEntry* list;
  hist_list_of(p, lists_ws, seg, &counts, &list);
  const int ntpb = (p.Bh + 31) / 32;
  if (p.D == 64)
    HGA_LAUNCH(HGA_K_BWD_HIST, (dkdv_hist_kernel<64>), dim3(256), dim3(512), 0, st,
               (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, lse, (const __bf16*)dO,
               delta_seg, (const HistEntry*)list, (const int*)counts, a, maxd, ntpb);
  else
    HGA_LAUNCH(HGA_K_BWD_HIST, (dkdv_hist_kernel<128>), dim3(256), dim3(512), 0, st,
               (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, lse, (const __bf16*)dO,
               delta_seg, (const HistEntry*)list, (const int*)counts, a, maxd, ntpb);
  return hipGetLastError();
}
size_t bwd_partial_bytes(const Prob& p) { return partial_bytes(p); }

size_t bwd_exact_workspace_bytes(const Prob& p) {
  return delta_bytes(p) + partial_bytes(p) + hist_list_bytes(p);
}

hipError_t launch_bwd(const Prob& p, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, const int32_t* sel,
                      int seg, void* dq, void* dk, void* dv, float* delta_ws, hipStream_t st,
                      bool delta_ready, float* hist_dk, float* hist_dv, float* partials) {
  // the f32 kernels and the exact gradient read full-sequence K / V only
  if ((p.dtype != HGA_BF16 || hist_dk != nullptr) && p.kv_rows != p.S)
    return hipErrorInvalidValue;
  if (p.dtype == HGA_BF16)
    return p.D == 64 ? bwd_bf16<64>(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, delta_ws, st,
                                    delta_ready, hist_dk, hist_dv, partials)
                     : bwd_bf16<128>(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, delta_ws, st,
                                     delta_ready, hist_dk, hist_dv, partials);
  return p.D == 64 ? bwd_f32<64>(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, delta_ws, st)
                   : bwd_f32<128>(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, delta_ws, st);
}

}  // namespace hga
