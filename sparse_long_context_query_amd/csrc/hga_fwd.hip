// a5: HGA forward attention of one segment, gfx950.
//
// [JA] 背景と概要 (also [DE] Hintergrund, [KO] 배경): instead of dense
// attention over the whole history, each query block attends to a bounded,
// exact set of history tokens; together with the active segment this keeps
// the per-token cost roughly constant in the total length.  [FR] Contexte:
// the bounded set is loaded in a targeted way per query block.
//
// For query token t of head h (KV head g = h/G, query block j) the keys are
// the tokens of the blocks selected for (b, g, j) and the local tokens
// t0..t.  One softmax over that joint set: o = sum p v, lse = log sum exp.
#include <hip/hip_runtime.h>

#include "hga_internal.h"
#include "hga_tiles.h"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct FwdArgs {
  int B, S, L, Bh, Bq, K, Hq, Hkv, G, nqb, nqb_all, seg;
  int nseg;   // segments seg .. seg+nseg-1 in one launch (whole-pass kernel)
  int wpu;    // blocks of threads per (b, g, j) unit
  int nq32;   // 32-row query sub-blocks per query block
  float c2;   // softmax scale * log2(e)
  int dchunk; // whole-pass kernel: floats between the delta rows of two segments
  int Skv;    // step kernel: K/V rows per (b, g)
  int kv_t0;  // step kernel: K/V row of the segment's first key
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  512 threads = 8 waves.  A block of threads owns up to 4
// "wave rows" of one (b, g, j) unit (a wave row = 32 query tokens of one
// head: query sub-block qs, head hh of the group), so all its waves share
// one key set.  The key tiles (64 keys; history tiles first, then local
// tiles) are split in two halves: waves 0-3 walk the first half and waves
// 4-7 the second, two waves per SIMD so that one wave's softmax overlaps
// the other's MFMAs.  Each half double-buffers its tiles in LDS; the next
// tile's K and V rows are copied straight from memory into swizzled
// row-major LDS tiles while the current tile is computed.  Per wave and
// tile: S^T = K.Q^T (Q^T held in registers as B operand), online softmax
// per query, O^T += V^T.P^T with V^T read transposed from the V tile and P^T
// taken from the accumulator.  The running max is only raised when a tile
// max exceeds it by more than kRescale (log2 units), so O is rarely
// rescaled; exp2 arguments stay below kRescale and the final normalisation
// is exact either way.  The halves' partial (O, m, l) are merged through
// LDS at the end (log-sum-exp rule).
// ---------------------------------------------------------------------------
constexpr float kRescale = 8.f;

template <int D>
__global__ __launch_bounds__(512) void fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const int32_t* __restrict__ sel,
    __bf16* __restrict__ o, float* __restrict__ lse, const __bf16* __restrict__ dO,
    float* __restrict__ delta, FwdArgs a) {
  constexpr int TK = 64;
  constexpr int NKK = D / 16;  // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int TILE_B = TK * 2 * D;
  constexpr int STAGE_B = 2 * TILE_B;  // K tile + V tile
  static_assert(4 * STAGE_B >= 4 * (NDB * 16 * 64 + 2 * 64) * 4, "merge buffer fits");

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

  // the query rows do not depend on the selection: request them first so
  // that their latency overlaps the compaction
  const int tq = qfirst + lq;
  const bool row_ok = lq < nvalid;
  bf16x8 qreg[NKK];
  {
    const __bf16* qp = q + ((size_t)(b * a.Hq + h) * a.S + tq) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qreg[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * kk) : bf16x8{};
  }

  const int32_t* srow = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)a.seg * a.nqb + j) * a.K;
  const int nsel = compact_selection(srow, a.K, nb, s_hlist, &s_hcount);
  KeySource<TK> src;
  src.init(s_hlist, nsel, a.Bh, a.kv_t0, a.kv_t0 + a.L);  // K/V rows, not tokens
  const int ntiles = src.n_hist_tiles + (blk_qmax - t0) / TK + 1;
  const int n0 = (ntiles + 1) / 2;              // tiles of half 0
  const int my_first = half ? n0 : 0;
  const int my_count = half ? ntiles - n0 : n0;

  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.Skv * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kv_base, (uint32_t)a.Skv * (2 * D));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + kv_base, (uint32_t)a.Skv * (2 * D));
  const __amdgpu_buffer_rsrc_t kr_none = make_rsrc(k + kv_base, 0u);
  const __amdgpu_buffer_rsrc_t vr_none = make_rsrc(v + kv_base, 0u);


  floatx16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;
  FragOffsets<D> fo;
  fo.init(lane);

  if (my_count > 0)
    dma_kv_tile<D, TK>(src, my_first, kr, vr, s_tiles[half][0], s_tiles[half][0] + TILE_B, wr,
                       lane);
  drain_vmem_loads();
  __syncthreads();

  for (int i = 0; i < n0; ++i) {
    const int it = my_first + i;
    const bool mine = i < my_count;
    // the next tile's copies: offsets now, issue among the score MFMAs (an
    // empty resource when there is no next tile)
    const bool copy_next = i + 1 < my_count;
    uint32_t coff[TK / (64 / ((2 * D) / 16)) / 4];
    kv_tile_offsets<D, TK>(src, copy_next ? it + 1 : it, wr, lane, coff);
    const __amdgpu_buffer_rsrc_t kr_n = copy_next ? kr : kr_none;
    const __amdgpu_buffer_rsrc_t vr_n = copy_next ? vr : vr_none;
    unsigned char* const knext = s_tiles[half][(i + 1) & 1];

    const bool is_local = it >= src.n_hist_tiles;
    const int local_first = t0 + (it - src.n_hist_tiles) * TK;
    const bool work = mine && active && (!is_local || local_first <= wave_qmax);
    if (!work) kv_tile_issue<D, TK>(kr_n, vr_n, coff, knext, knext + TILE_B, wr);
    if (work) {
      const unsigned char* kt = s_tiles[half][i & 1];
      const unsigned char* vt = kt + TILE_B;
      // all K fragments of the tile are requested before the first MFMA so
      // that the LDS latency is paid once per tile, not once per k-step
      bf16x8 kf[NKK][2];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int st = 0; st < 2; ++st) kf[kk][st] = fo.row(kt, st, kk);
      floatx16 sacc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) sacc[st] = floatx16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int st = 0; st < 2; ++st) sacc[st] = mfma32(kf[kk][st], qreg[kk], sacc[st]);
      }
      kv_tile_issue<D, TK>(kr_n, vr_n, coff, knext, knext + TILE_B, wr);
      // keep that order through instruction scheduling: 2*NKK LDS reads, then
      // the MFMAs with the copies spread among them
      constexpr int NCP = 2 * (TK / (64 / ((2 * D) / 16)) / 4);  // copy instructions
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKK, 0);
#pragma unroll
      for (int u = 0; u < NCP; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NKK / NCP, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      // tile max of the raw scores; mask only on tiles that can hold
      // invisible keys
      const bool need_mask = is_local ? (local_first + TK - 1 > qfirst)
                                      : ((it + 1) * TK > src.nh);
      if (need_mask) {
        const int base = is_local ? local_first : it * TK;
        const int lim = is_local ? tq : src.nh - 1;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr_ = base + 32 * st + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (kr_ > lim) sacc[st][r] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[st][r]);
      mt = pair_max(mt) * a.c2;
      const bool raise = mt > m_run + kRescale;
      if (__ballot(raise)) {
        const float m_new = raise ? mt : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[st][r], a.c2, -m_use));
          sacc[st][r] = p;
          rs += p;
        }
      }
      l_run += rs;  // this lane's 32 keys; the partner lane's are added at the end
      // O^T += V^T . P^T
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 8 * ks;
          const bf16x8 pb = to_bf16x8(sacc[st][r0], sacc[st][r0 + 1], sacc[st][r0 + 2],
                                      sacc[st][r0 + 3], sacc[st][r0 + 4], sacc[st][r0 + 5],
                                      sacc[st][r0 + 6], sacc[st][r0 + 7]);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            oacc[db] = mfma32(fo.tr(vt, 32 * st + 16 * ks, db), pb, oacc[db]);
        }
      }
    }
    drain_vmem_loads();  // the next tile has landed in LDS
    __syncthreads();
  }

  // both lanes of a query kept partial row sums over their own keys
  l_run = pair_sum(l_run);

  // fused delta: the dO elements this lane multiplies are requested now, so
  // that their latency overlaps the merge below
  const size_t orow = ((size_t)(b * a.Hq + h) * a.S + tq) * D;
  const bool want_delta = delta != nullptr && half == 0 && active && row_ok;
  bf16x4 dog[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      dog[db][r4] = want_delta
                        ? *reinterpret_cast<const bf16x4*>(dO + orow + 32 * db + 8 * r4 + 4 * hi)
                        : bf16x4{};

  // merge the two halves: half 1 parks (m, l, O^T) in LDS, half 0 combines
  float* park = reinterpret_cast<float*>(&s_tiles[0][0][0]);
  float4* park_o = reinterpret_cast<float4*>(park) + wr * (NDB * 4 * 64);
  float* park_ml = park + 4 * (NDB * 16 * 64) + wr * 128;
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        park_o[(db * 4 + r4) * 64 + lane] = make_float4(oacc[db][4 * r4], oacc[db][4 * r4 + 1],
                                                        oacc[db][4 * r4 + 2], oacc[db][4 * r4 + 3]);
    park_ml[lane] = m_run;
    park_ml[64 + lane] = l_run;
  }
  __syncthreads();
  if (half == 0 && active && row_ok) {
    const float m1 = park_ml[lane], l1 = park_ml[64 + lane];
    const float m = fmaxf(m_run, m1);
    const float f0 = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m);
    const float f1 = (m1 == -INFINITY) ? 0.f : exp2f(m1 - m);
    const float l = l_run * f0 + l1 * f1;
    const float inv = 1.f / l;
    const float g0 = f0 * inv, g1 = f1 * inv;
    __bf16* op = o + orow;
    float dsum = 0.f;  // this lane's half of rowsum(dO * o) (fused delta)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 p4 = park_o[(db * 4 + r4) * 64 + lane];
        const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(oacc[db][4 * r4 + e] * g0 + pv[e] * g1);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * r4 + 4 * hi) = pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) dsum += (float)pk[e] * (float)dog[db][r4][e];
      }
    }
    if (lse != nullptr && hi == 0)
      lse[(size_t)(b * a.Hq + h) * a.S + tq] = (m + log2f(l)) * kLn2;
    if (delta != nullptr) {
      // delta of the stored (rounded) o, as the separate delta pass computes it
      dsum = pair_sum(dsum);
      if (hi == 0) delta[(size_t)(b * a.Hq + h) * a.L + (tq - t0)] = dsum;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel for a whole segmented pass (segments a.seg .. a.seg +
// a.nseg - 1 in one launch).  Once the selections of every segment exist the
// segments are independent, so one grid holds all their query blocks and no
// key split is needed for parallelism: a block of 4 waves owns up to 4 wave
// rows of one (segment, b, g, j) unit and walks every key tile of that unit
// itself.  Two such blocks share a CU (64 KB of tiles each), and since they
// are not tied by a common barrier, one block's softmax and copies run while
// the other's MFMAs issue.  Per wave and tile the work is that of
// fwd_bf16_kernel; the final normalisation needs no merge.
//
// Work order: blocks are dealt to XCDs in contiguous ranges (xcd_remap), a
// range covering the units of one (b, g) so that they share an L2; inside
// it the segments run from the last to the first and the query blocks from
// the last to the first, the units with the most keys first, so that the
// launch ends on short units.
//
// delta (with dO): row sums of dO * o, segment s's [B, Hq, L] rows at
// delta + (s - a.seg) * a.dchunk.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void fwd_pass_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const int32_t* __restrict__ sel,
    __bf16* __restrict__ o, float* __restrict__ lse, const __bf16* __restrict__ dO,
    float* __restrict__ delta, FwdArgs a) {
  constexpr int TK = 64;
  constexpr int NKK = D / 16;  // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
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
  const int seg = a.seg + a.nseg - 1 - w % a.nseg;
  w /= a.nseg;
  const int g = w % a.Hkv;
  const int b = w / a.Hkv;
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

  const int tq = qfirst + lq;
  const bool row_ok = lq < nvalid;
  bf16x8 qreg[NKK];
  {
    const __bf16* qp = q + ((size_t)(b * a.Hq + h) * a.S + tq) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qreg[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * kk) : bf16x8{};
  }

  const int32_t* srow = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)seg * a.nqb + j) * a.K;
  const int nsel = compact_selection(srow, a.K, nb, s_hlist, &s_hcount);
  KeySource<TK> src;
  src.init(s_hlist, nsel, a.Bh, t0, t0 + a.L);
  const int ntiles = src.n_hist_tiles + (blk_qmax - t0) / TK + 1;

  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kv_base, (uint32_t)a.S * (2 * D));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + kv_base, (uint32_t)a.S * (2 * D));
  const __amdgpu_buffer_rsrc_t kr_none = make_rsrc(k + kv_base, 0u);
  const __amdgpu_buffer_rsrc_t vr_none = make_rsrc(v + kv_base, 0u);

  floatx16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;
  FragOffsets<D> fo;
  fo.init(lane);
  // when every tile is a run of consecutive rows (tpb > 0), the copies take
  // loop-invariant lane offsets inside a resource placed at the tile's first
  // row, built with scalar instructions per tile
  uint32_t loff[TK / (64 / ((2 * D) / 16)) / 4];
  contiguous_tile_offsets<D, TK>(wr, lane, loff);

  dma_kv_tile<D, TK>(src, 0, kr, vr, s_tiles[0], s_tiles[0] + TILE_B, wr, lane);
  drain_vmem_loads();
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const bool copy_next = it + 1 < ntiles;
    uint32_t coff[TK / (64 / ((2 * D) / 16)) / 4];
    __amdgpu_buffer_rsrc_t kr_n, vr_n;
    if (src.tpb > 0) {
      // rows past the segment end (last local tile) are read as they are
      // and masked; past the sequence end the resource returns zeros
      const int base = src.tile_base(copy_next ? it + 1 : it);
      const uint32_t nbytes = copy_next ? (uint32_t)(a.S - base) * (2 * D) : 0u;
      kr_n = make_rsrc(k + kv_base + (size_t)base * D, nbytes);
      vr_n = make_rsrc(v + kv_base + (size_t)base * D, nbytes);
#pragma unroll
      for (int n = 0; n < TK / (64 / ((2 * D) / 16)) / 4; ++n) coff[n] = loff[n];
    } else {
      kv_tile_offsets<D, TK>(src, copy_next ? it + 1 : it, wr, lane, coff);
      kr_n = copy_next ? kr : kr_none;
      vr_n = copy_next ? vr : vr_none;
    }
    unsigned char* const knext = s_tiles[(it + 1) & 1];

    const bool is_local = it >= src.n_hist_tiles;
    const int local_first = t0 + (it - src.n_hist_tiles) * TK;
    const bool work = active && (!is_local || local_first <= wave_qmax);
    if (!work) kv_tile_issue<D, TK>(kr_n, vr_n, coff, knext, knext + TILE_B, wr);
    if (work) {
      const unsigned char* kt = s_tiles[it & 1];
      const unsigned char* vt = kt + TILE_B;
      bf16x8 kf[NKK][2];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int st = 0; st < 2; ++st) kf[kk][st] = fo.row(kt, st, kk);
      floatx16 sacc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) sacc[st] = floatx16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int st = 0; st < 2; ++st) sacc[st] = mfma32(kf[kk][st], qreg[kk], sacc[st]);
      }
      kv_tile_issue<D, TK>(kr_n, vr_n, coff, knext, knext + TILE_B, wr);
      constexpr int NCP = 2 * (TK / (64 / ((2 * D) / 16)) / 4);  // copy instructions
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKK, 0);
#pragma unroll
      for (int u = 0; u < NCP; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NKK / NCP, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      const bool need_mask = is_local ? (local_first + TK - 1 > qfirst)
                                      : ((it + 1) * TK > src.nh);
      if (need_mask) {
        const int base = is_local ? local_first : it * TK;
        const int lim = is_local ? tq : src.nh - 1;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr_ = base + 32 * st + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (kr_ > lim) sacc[st][r] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[st][r]);
      mt = pair_max(mt) * a.c2;
      const bool raise = mt > m_run + kRescale;
      if (__ballot(raise)) {
        const float m_new = raise ? mt : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[st][r], a.c2, -m_use));
          sacc[st][r] = p;
          rs += p;
        }
      }
      l_run += rs;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 8 * ks;
          const bf16x8 pb = to_bf16x8(sacc[st][r0], sacc[st][r0 + 1], sacc[st][r0 + 2],
                                      sacc[st][r0 + 3], sacc[st][r0 + 4], sacc[st][r0 + 5],
                                      sacc[st][r0 + 6], sacc[st][r0 + 7]);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            oacc[db] = mfma32(fo.tr(vt, 32 * st + 16 * ks, db), pb, oacc[db]);
        }
      }
    }
    drain_vmem_loads();  // the next tile has landed in LDS
    __syncthreads();
  }

  if (!(active && row_ok)) return;
  l_run = pair_sum(l_run);
  const size_t orow = ((size_t)(b * a.Hq + h) * a.S + tq) * D;
  const bool want_delta = delta != nullptr;
  bf16x4 dog[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      dog[db][r4] = want_delta
                        ? *reinterpret_cast<const bf16x4*>(dO + orow + 32 * db + 8 * r4 + 4 * hi)
                        : bf16x4{};
  const float inv = 1.f / l_run;
  __bf16* op = o + orow;
  float dsum = 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(oacc[db][4 * r4 + e] * inv);
      *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * r4 + 4 * hi) = pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) dsum += (float)pk[e] * (float)dog[db][r4][e];
    }
  }
  if (lse != nullptr && hi == 0)
    lse[(size_t)(b * a.Hq + h) * a.S + tq] = (m_run + log2f(l_run)) * kLn2;
  if (want_delta) {
    dsum = pair_sum(dsum);
    if (hi == 0)
      delta[(size_t)(seg - a.seg) * a.dchunk + (size_t)(b * a.Hq + h) * a.L + (tq - t0)] = dsum;
  }
}

// ---------------------------------------------------------------------------
// float32 kernel (reference-precision path; plain VALU).  One wave per
// (b, h, 64-query chunk of a query block); one query per lane; key tiles of
// 32 rows staged in LDS and broadcast to the lanes.  Online softmax per key
// in natural-log units.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const int32_t* __restrict__ sel,
    float* __restrict__ o, float* __restrict__ lse, FwdArgs a, float scale) {
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

  float qr[D], acc[D];
  const float* qp = q + ((size_t)(b * a.Hq + h) * a.S + tq) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) { qr[d] = qp[d]; acc[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
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
      if (slot >= nh && t0 + (slot - nh) > tq) continue;  // causal
      float z = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) z += qr[d] * s_k[r][d];
      z *= scale;
      if (z > m) {
        const float al = expf(m - z);
        l *= al;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= al;
        m = z;
      }
      const float p = expf(z - m);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] += p * s_v[r][d];
    }
    __syncthreads();
  }
  if (row_ok) {
    float* op = o + ((size_t)(b * a.Hq + h) * a.S + tq) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
    if (lse != nullptr) lse[(size_t)(b * a.Hq + h) * a.S + tq] = m + logf(l);
  }
}

FwdArgs make_args(const Prob& p, int seg) {
  FwdArgs a;
  a.S = p.S; a.L = p.L; a.Bh = p.Bh; a.Bq = p.Bq; a.K = p.K; a.Hq = p.Hq; a.Hkv = p.Hkv;
  a.G = p.G; a.nqb = p.nqb; a.nqb_all = p.nqb_all; a.seg = seg;
  a.B = p.B; a.nseg = 1; a.dchunk = 0;
  a.Skv = p.kv_rows;
  a.kv_t0 = p.kv_local >= 0 ? p.kv_local : seg * p.L;
  a.nq32 = (p.Bq + 31) / 32;
  a.wpu = (p.G * a.nq32 + 3) / 4;
  a.c2 = p.scale * kLog2e;
  return a;
}

template <int D>
hipError_t fwd_pass_bf16(const Prob& p, const void* q, const void* k, const void* v,
                         const int32_t* sel, int seg0, int nseg, void* o, float* lse,
                         hipStream_t st, const void* dO, float* delta, size_t delta_stride) {
  FwdArgs a = make_args(p, seg0);
  a.nseg = nseg;
  a.dchunk = (int)(delta_stride / sizeof(float));
  const int nblocks = p.B * p.Hkv * nseg * p.nqb * a.wpu;
  HGA_LAUNCH(HGA_K_FWD, (fwd_pass_kernel<D>), dim3(nblocks), dim3(256), 0, st,
             (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, sel, (__bf16*)o, lse,
             (const __bf16*)dO, delta, a);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_bf16(const Prob& p, const void* q, const void* k, const void* v,
                    const int32_t* sel, int seg, void* o, float* lse, hipStream_t st,
                    const void* dO, float* delta) {
  FwdArgs a = make_args(p, seg);
  const int nblocks = p.B * p.Hkv * p.nqb * a.wpu;
  HGA_LAUNCH(HGA_K_FWD, (fwd_bf16_kernel<D>), dim3(nblocks), dim3(512), 0, st,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, sel, (__bf16*)o,
                     lse, (const __bf16*)dO, delta, a);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_f32(const Prob& p, const void* q, const void* k, const void* v,
                   const int32_t* sel, int seg, void* o, float* lse, hipStream_t st) {
  FwdArgs a = make_args(p, seg);
  const int nblocks = p.B * p.Hq * p.nqb * ((p.Bq + 63) / 64);
  HGA_LAUNCH(HGA_K_FWD, (fwd_f32_kernel<D>), dim3(nblocks), dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, sel, (float*)o, lse, a, p.scale);
  return hipGetLastError();
}

}  // namespace

bool fused_delta(const Prob& p) { return p.dtype == HGA_BF16; }

hipError_t launch_fwd_pass(const Prob& p, const void* q, const void* k, const void* v,
                           const int32_t* sel, int seg0, int nseg, void* o, float* lse,
                           hipStream_t st, const void* dO, float* delta, size_t delta_stride) {
  if (p.dtype != HGA_BF16 || p.kv_rows != p.S) return hipErrorInvalidValue;
  if (dO == nullptr) delta = nullptr;
  return p.D == 64 ? fwd_pass_bf16<64>(p, q, k, v, sel, seg0, nseg, o, lse, st, dO, delta,
                                       delta_stride)
                   : fwd_pass_bf16<128>(p, q, k, v, sel, seg0, nseg, o, lse, st, dO, delta,
                                        delta_stride);
}

hipError_t launch_fwd(const Prob& p, const void* q, const void* k, const void* v,
                      const int32_t* sel, int seg, void* o, float* lse, hipStream_t st,
                      const void* dO, float* delta) {
  if (dO == nullptr || !fused_delta(p)) delta = nullptr;
  if (p.dtype != HGA_BF16 && p.kv_rows != p.S) return hipErrorInvalidValue;
  if (p.dtype == HGA_BF16)
    return p.D == 64 ? fwd_bf16<64>(p, q, k, v, sel, seg, o, lse, st, dO, delta)
                     : fwd_bf16<128>(p, q, k, v, sel, seg, o, lse, st, dO, delta);
  return p.D == 64 ? fwd_f32<64>(p, q, k, v, sel, seg, o, lse, st)
                   : fwd_f32<128>(p, q, k, v, sel, seg, o, lse, st);
}

}  // namespace hga
