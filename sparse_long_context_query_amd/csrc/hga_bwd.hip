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

#include "hga_internal.h"
#include "hga_tiles.h"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
  int S, L, Bh, Bq, K, Hq, Hkv, G, nqb, nqb_all, seg;
  int wpu;      // dq: blocks of threads per (b, g, j) unit
  int nq32;     // 32-row query sub-blocks per query block
  float c2;     // scale * log2(e)
  float scale;
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

// ---------------------------------------------------------------------------
// a7, bf16 MFMA: dq.  Same work split as the forward: 512 threads = 8 waves,
// up to 4 wave rows (32 queries of one head each) of one (b, g, j) unit per
// block of threads; the key tiles (64 keys) are split in two halves walked
// by waves 0-3 and 4-7, each half double-buffering swizzled row-major K
// and V tiles that are copied straight from memory into LDS.  Per wave and
// 32-key sub-tile:
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
    const int32_t* __restrict__ sel, __bf16* __restrict__ dq, BwdArgs a) {
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

  const int32_t* srow = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)a.seg * a.nqb + j) * a.K;
  const int nsel = compact_selection(srow, a.K, nb, s_hlist, &s_hcount);
  KeySource<TK> src;
  src.init(s_hlist, nsel, a.Bh, t0, t0 + a.L);
  const int ntiles = src.n_hist_tiles + (blk_qmax - t0) / TK + 1;
  const int n0 = (ntiles + 1) / 2;
  const int my_first = half ? n0 : 0;
  const int my_count = half ? ntiles - n0 : n0;

  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kv_base, (uint32_t)a.S * (2 * D));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + kv_base, (uint32_t)a.S * (2 * D));

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

  floatx16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = floatx16{};
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
    if (i + 1 < my_count)
      dma_kv_tile<D, TK>(src, it + 1, kr, vr, s_tiles[half][(i + 1) & 1],
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
        floatx16 sacc = floatx16{}, pacc = floatx16{};
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
          sacc[r] = p * (pacc[r] - dlt);
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
  float* park = reinterpret_cast<float*>(&s_tiles[0][0][0]) + wr * (NDB * 16 * 64);
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) park[(db * 16 + r) * 64 + lane] = dqacc[db][r];
  }
  __syncthreads();
  if (half == 0 && active && row_ok) {
    __bf16* op = dq + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          pk[e] = (__bf16)((dqacc[db][r] + park[(db * 16 + r) * 64 + lane]) * a.scale);
        }
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * r4 + 4 * hi) = pk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// a8, bf16 MFMA: dk/dv of the local keys.  One block of threads (8 waves)
// per (b, g, 32-key tile kt of the segment).  The (query head, 32-query
// tile) pairs that see the key tile (query tiles kt.. of every head of the
// group) are dealt round-robin to the 8 waves, two per SIMD, so one wave's
// loads and softmax overlap the other's MFMAs.  A wave copies its pair's Q
// and dO tiles and their lse / delta straight from memory into its own
// swizzled LDS slice (no register staging), then, with the key tile's K
// and V rows held in registers as B operands:
//   S  = Q . K^T,  dP = dO . V^T      (A operands: tile rows)
//   P  = exp2(S c2 - lse2), dS = P * (dP - delta)
//   dV^T += dO^T . P,  dK^T += Q^T . dS   (A operands: transposed reads of
//                                          the same tiles)
// The 8 partial dK^T, dV^T are folded pairwise through LDS at the end.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512) void dkdv_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, BwdArgs a) {
  constexpr int TQ = 32;                 // queries per tile
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE_B = TQ * 2 * D;     // bytes of one row-major tile
  constexpr int SLICE_B = 2 * TILE_B + 256;  // Q tile, dO tile, lse + delta
  constexpr int NW = 8;
  constexpr int PART_F = 2 * NDB * 16 * 64;  // floats of one wave's (dK^T, dV^T)
  constexpr int STAGE_B = 2 * TILE_B + NW * SLICE_B;  // K, V tiles + wave slices
  constexpr int LDS_BYTES = STAGE_B > 4 * PART_F * 4 ? STAGE_B : 4 * PART_F * 4;
  __shared__ __attribute__((aligned(1024))) unsigned char s_raw[LDS_BYTES];

  const int nkt = (a.L + 31) / 32;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = w % nkt;
  const int g = (w / nkt) % a.Hkv;
  const int b = w / (nkt * a.Hkv);
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

  // K and V rows of this key tile, shared by the 8 waves as B operands
  // (lane (key lq, hi) reads K[key][16kk + 8hi .. +7])
  const int kfirst = t0 + kt * 32;
  const int tk = kfirst + lq;
  const bool key_ok = tk < tend;
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;
  if (wave == 0) dma_rows<D>(k + kv_base + (size_t)kfirst * D, 32, tend - kfirst, s_k, lane);
  if (wave == 1) dma_rows<D>(v + kv_base + (size_t)kfirst * D, 32, tend - kfirst, s_v, lane);
  drain_vmem_loads();
  __syncthreads();

  floatx16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkacc[db] = floatx16{}; dvacc[db] = floatx16{}; }
  FragOffsets<D> fo;
  fo.init(lane);

  const int nqt = (a.L + TQ - 1) / TQ;
  const int npairs = (nqt - kt) * a.G;
  for (int pi = wave; pi < npairs; pi += NW) {
    const int qt = kt + pi / a.G;
    const int h = g * a.G + pi % a.G;
    const int tq0 = t0 + qt * TQ;
    const size_t hrow = (size_t)(b * a.Hq + h) * a.S;
    const int nvalid = min(TQ, tend - tq0);
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
    // C layout: lane = key lq, item r = query row 8(r/4)+4hi+(r%4) of the tile
    const bool need_mask = (tq0 < kfirst + 31) || (nvalid < TQ) || (kfirst + 32 > tend);
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
          const int tqr = tq0 + 8 * r4 + 4 * hi + e;
          p = (key_ok && tk <= tqr && tqr < tend) ? p : 0.f;
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

  // fold the 8 partial sums pairwise through LDS: 8 -> 4 -> 2 -> 1 (the
  // first barrier also retires every wave's reads of the K/V tiles)
  float* fold = reinterpret_cast<float*>(s_raw);
  for (int span = NW / 2; span >= 1; span >>= 1) {
    __syncthreads();
    if (wave >= span && wave < 2 * span) {
      float* dst = fold + (wave - span) * PART_F;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dst[((0 * NDB + db) * 16 + r) * 64 + lane] = dkacc[db][r];
          dst[((1 * NDB + db) * 16 + r) * 64 + lane] = dvacc[db][r];
        }
    }
    __syncthreads();
    if (wave < span) {
      const float* src_ = fold + wave * PART_F;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dkacc[db][r] += src_[((0 * NDB + db) * 16 + r) * 64 + lane];
          dvacc[db][r] += src_[((1 * NDB + db) * 16 + r) * 64 + lane];
        }
    }
  }
  if (wave == 0 && key_ok) {
    __bf16* kp = dk + kv_base + (size_t)tk * D;
    __bf16* vp = dv + kv_base + (size_t)tk * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 pk, pw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[e] = (__bf16)(dkacc[db][4 * r4 + e] * a.scale);
          pw[e] = (__bf16)(dvacc[db][4 * r4 + e]);
        }
        *reinterpret_cast<bf16x4*>(kp + 32 * db + 8 * r4 + 4 * hi) = pk;
        *reinterpret_cast<bf16x4*>(vp + 32 * db + 8 * r4 + 4 * hi) = pw;
      }
    }
  }
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
  a.S = p.S; a.L = p.L; a.Bh = p.Bh; a.Bq = p.Bq; a.K = p.K; a.Hq = p.Hq; a.Hkv = p.Hkv;
  a.G = p.G; a.nqb = p.nqb; a.nqb_all = p.nqb_all; a.seg = seg;
  a.nq32 = (p.Bq + 31) / 32;
  a.wpu = (p.G * a.nq32 + 3) / 4;
  a.c2 = p.scale * kLog2e;
  a.scale = p.scale;
  return a;
}

template <typename T, int D>
hipError_t delta_t(const Prob& p, const void* o, const void* dO, int seg, float* delta,
                   hipStream_t st) {
  constexpr int C = D / Vec16<T>::N;
  constexpr int RPB = 256 / C;
  const int nrows = p.B * p.Hq * p.L;
  ProfScope ps(HGA_K_BWD_PRE, st);
  hipLaunchKernelGGL((delta_kernel<T, D>), dim3((nrows + RPB - 1) / RPB), dim3(256), 0, st,
                     (const T*)o, (const T*)dO, delta, p.S, p.L, seg * p.L, nrows);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_bf16(const Prob& p, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dO, const int32_t* sel,
                    int seg, void* dq, void* dk, void* dv, float* delta, hipStream_t st) {
  hipError_t e = delta_t<__bf16, D>(p, o, dO, seg, delta, st);
  if (e != hipSuccess) return e;
  BwdArgs a = make_args(p, seg);
  {
    const int nblocks = p.B * p.Hkv * p.nqb * a.wpu;
    ProfScope ps(HGA_K_BWD_DQ, st);
    hipLaunchKernelGGL((dq_bf16_kernel<D>), dim3(nblocks), dim3(512), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, lse, (const __bf16*)dO, delta, sel,
                       (__bf16*)dq, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nblocks = p.B * p.Hkv * ((p.L + 31) / 32);
    ProfScope ps(HGA_K_BWD_DKDV, st);
    hipLaunchKernelGGL((dkdv_bf16_kernel<D>), dim3(nblocks), dim3(512), 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, lse,
                       (const __bf16*)dO, delta, (__bf16*)dk, (__bf16*)dv, a);
    e = hipGetLastError();
  }
  return e;
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
    ProfScope ps(HGA_K_BWD_DQ, st);
    hipLaunchKernelGGL((dq_f32_kernel<D>), dim3(nblocks), dim3(64), 0, st, (const float*)q,
                       (const float*)k, (const float*)v, lse, (const float*)dO, delta, sel,
                       (float*)dq, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nblocks = p.B * p.Hkv * ((p.L + 63) / 64);
    ProfScope ps(HGA_K_BWD_DKDV, st);
    hipLaunchKernelGGL((dkdv_f32_kernel<D>), dim3(nblocks), dim3(64), 0, st, (const float*)q,
                       (const float*)k, (const float*)v, lse, (const float*)dO, delta,
                       (float*)dk, (float*)dv, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

size_t bwd_workspace_bytes(const Prob& p) {
  const size_t delta = (size_t)p.B * p.Hq * p.L * sizeof(float);
  return (delta + 255) & ~(size_t)255;
}

hipError_t launch_bwd(const Prob& p, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, const int32_t* sel,
                      int seg, void* dq, void* dk, void* dv, float* delta_ws, hipStream_t st) {
  if (p.dtype == HGA_BF16)
    return p.D == 64 ? bwd_bf16<64>(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, delta_ws, st)
                     : bwd_bf16<128>(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, delta_ws, st);
  return p.D == 64 ? bwd_f32<64>(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, delta_ws, st)
                   : bwd_f32<128>(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, delta_ws, st);
}

}  // namespace hga
