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
  int S, L, Bh, Bq, K, Hq, Hkv, G, nqb, nqb_all, seg;
  int wpu;    // blocks of threads per (b, g, j) unit
  int nq32;   // 32-row query sub-blocks per query block
  float c2;   // softmax scale * log2(e)
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  256 threads = 4 waves; each wave owns 32 query rows of
// one head (a "wave row": query sub-block qs of 32 tokens, head hh of the
// group); the waves of a block of threads share one (b, g, j) unit and so
// one key set, which is staged through LDS in 64-key tiles (K row-major,
// V transposed), double buffered with the next tile's global loads in
// registers.  Per wave and tile: S^T = K.Q^T (keys x queries, Q^T held in
// registers as the B operand), online softmax per query (one query per
// lane pair), O^T += V^T.P^T with P^T fed straight from the accumulator.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const int32_t* __restrict__ sel,
    __bf16* __restrict__ o, float* __restrict__ lse, FwdArgs a) {
  constexpr int TK = 64;
  using G_ = TileGeom<D, TK>;
  constexpr int KSTR = G_::KSTR;
  constexpr int NKK = D / 16;  // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int JOB_C = D / 8;

  __shared__ __bf16 s_k[2][G_::ROW_ELEMS];
  __shared__ __bf16 s_vt[2][G_::T_ELEMS];
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
  const int wave = tid >> 6, lane = tid & 63, lq = lane & 31, hi = lane >> 5;

  // wave row of this wave and the block's last query token
  const int nwr = a.G * a.nq32;
  const int idx = c * 4 + wave;
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

  // selected history blocks of this unit
  const int32_t* srow = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)a.seg * a.nqb + j) * a.K;
  const int nsel = compact_selection(srow, a.K, nb, s_hlist, &s_hcount);
  KeySource<TK> src;
  src.init(s_hlist, nsel, a.Bh, t0, t0 + a.L);
  const int n_local_tiles = (blk_qmax - t0) / TK + 1;
  const int ntiles = src.n_hist_tiles + n_local_tiles;

  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;
  const __bf16* kg = k + kv_base;
  const __bf16* vg = v + kv_base;

  // Q^T as the B operand: lane (query lq, hi) holds Q[t][16kk+8hi .. +7]
  const int tq = qfirst + lq;
  const bool row_ok = lq < nvalid;
  bf16x8 qreg[NKK];
  {
    const __bf16* qp = q + ((size_t)(b * a.Hq + h) * a.S + tq) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (row_ok) qreg[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
      else qreg[kk] = bf16x8{};
    }
  }

  // staging: job = (4-row group rq, 8-dim chunk cc)
  const bool has_job = tid < G_::NJOB;
  const int rq = tid / JOB_C, cc = tid % JOB_C;
  uint4 kr[4], vr[4];
  auto load_tile = [&](int it) {
    if (!has_job) return;
    const int tok = src.token4(it, 4 * rq);
    if (tok < 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { kr[i] = make_uint4(0, 0, 0, 0); vr[i] = kr[i]; }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = *reinterpret_cast<const uint4*>(kg + (size_t)(tok + i) * D + 8 * cc);
      vr[i] = *reinterpret_cast<const uint4*>(vg + (size_t)(tok + i) * D + 8 * cc);
    }
  };
  auto store_tile = [&](int buf) {
    if (!has_job) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&s_k[buf][(4 * rq + i) * KSTR + 8 * cc]) = kr[i];
    const int pos = tpos(4 * rq);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint2*>(&s_vt[buf][toff<TK>(8 * cc + e, pos)]) =
          quad_column(vr[0], vr[1], vr[2], vr[3], e);
  };

  floatx16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) load_tile(it + 1);

    const bool is_local = it >= src.n_hist_tiles;
    const int local_first = t0 + (it - src.n_hist_tiles) * TK;
    const bool work = active && (!is_local || local_first <= wave_qmax);
    if (work) {
      const __bf16* kt = s_k[buf];
      const __bf16* vt = s_vt[buf];
      floatx16 sacc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        sacc[st] = floatx16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          sacc[st] = mfma32(lds_b128(kt + (32 * st + lq) * KSTR + 16 * kk + 8 * hi), qreg[kk],
                            sacc[st]);
      }
      // scale + mask, tile max per query
      const int hist_first = it * TK;
      float mt = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr_ = 32 * st + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = is_local ? (local_first + kr_ <= tq) : (hist_first + kr_ < src.nh);
          const float x = ok ? sacc[st][r] * a.c2 : -INFINITY;
          sacc[st][r] = x;
          mt = fmaxf(mt, x);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(sacc[st][r] - m_use);
          sacc[st][r] = p;
          rs += p;
        }
      }
      rs += __shfl_xor(rs, 32, 64);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      // O^T += V^T . P^T
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 8 * ks;
          const bf16x8 pb = to_bf16x8(sacc[st][r0], sacc[st][r0 + 1], sacc[st][r0 + 2],
                                      sacc[st][r0 + 3], sacc[st][r0 + 4], sacc[st][r0 + 5],
                                      sacc[st][r0 + 6], sacc[st][r0 + 7]);
          const int pos = 32 * st + 16 * ks + 8 * hi;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            oacc[db] = mfma32(lds_b128(vt + toff<TK>(32 * db + lq, pos)), pb, oacc[db]);
        }
      }
    }

    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (active && row_ok) {
    const float inv = 1.f / l_run;
    __bf16* op = o + ((size_t)(b * a.Hq + h) * a.S + tq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 pk;
        pk[0] = (__bf16)(oacc[db][4 * r4 + 0] * inv);
        pk[1] = (__bf16)(oacc[db][4 * r4 + 1] * inv);
        pk[2] = (__bf16)(oacc[db][4 * r4 + 2] * inv);
        pk[3] = (__bf16)(oacc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * r4 + 4 * hi) = pk;
      }
    }
    if (lse != nullptr && hi == 0)
      lse[(size_t)(b * a.Hq + h) * a.S + tq] = (m_run + log2f(l_run)) * kLn2;
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
  a.nq32 = (p.Bq + 31) / 32;
  a.wpu = (p.G * a.nq32 + 3) / 4;
  a.c2 = p.scale * kLog2e;
  return a;
}

template <int D>
hipError_t fwd_bf16(const Prob& p, const void* q, const void* k, const void* v,
                    const int32_t* sel, int seg, void* o, float* lse, hipStream_t st) {
  FwdArgs a = make_args(p, seg);
  const int nblocks = p.B * p.Hkv * p.nqb * a.wpu;
  ProfScope ps(HGA_K_FWD, st);
  hipLaunchKernelGGL((fwd_bf16_kernel<D>), dim3(nblocks), dim3(256), 0, st,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, sel, (__bf16*)o,
                     lse, a);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_f32(const Prob& p, const void* q, const void* k, const void* v,
                   const int32_t* sel, int seg, void* o, float* lse, hipStream_t st) {
  FwdArgs a = make_args(p, seg);
  const int nblocks = p.B * p.Hq * p.nqb * ((p.Bq + 63) / 64);
  ProfScope ps(HGA_K_FWD, st);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3(nblocks), dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, sel, (float*)o, lse, a, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const Prob& p, const void* q, const void* k, const void* v,
                      const int32_t* sel, int seg, void* o, float* lse, hipStream_t st) {
  if (p.dtype == HGA_BF16)
    return p.D == 64 ? fwd_bf16<64>(p, q, k, v, sel, seg, o, lse, st)
                     : fwd_bf16<128>(p, q, k, v, sel, seg, o, lse, st);
  return p.D == 64 ? fwd_f32<64>(p, q, k, v, sel, seg, o, lse, st)
                   : fwd_f32<128>(p, q, k, v, sel, seg, o, lse, st);
}

}  // namespace hga
