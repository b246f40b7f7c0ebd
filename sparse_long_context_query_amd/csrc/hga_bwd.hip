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
// a7, bf16 MFMA: dq.  Same work split as the forward (4 waves of 32 query
// rows sharing one (b, g, j) key set), 32-key tiles staged through LDS as
// K row-major, V row-major and K transposed.  Per wave and tile:
//   S^T  = K . Q^T          (Q^T in registers as B operand)
//   dP^T = V . dO^T         (dO^T in registers as B operand)
//   dS^T = P^T * (dP^T - delta),  P^T = exp2(S^T c2 - lse2)
//   dQ^T += K^T . dS^T      (dS^T straight from the accumulator)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void dq_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    const int32_t* __restrict__ sel, __bf16* __restrict__ dq, BwdArgs a) {
  constexpr int TK = 32;
  using G_ = TileGeom<D, TK>;
  constexpr int KSTR = G_::KSTR;
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int JOB_C = D / 8;

  __shared__ __bf16 s_k[2][G_::ROW_ELEMS];
  __shared__ __bf16 s_v[2][G_::ROW_ELEMS];
  __shared__ __bf16 s_kt[2][G_::T_ELEMS];
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

  const int32_t* srow = sel + ((size_t)(b * a.Hkv + g) * a.nqb_all + (size_t)a.seg * a.nqb + j) * a.K;
  const int nsel = compact_selection(srow, a.K, nb, s_hlist, &s_hcount);
  KeySource<TK> src;
  src.init(s_hlist, nsel, a.Bh, t0, t0 + a.L);
  const int ntiles = src.n_hist_tiles + (blk_qmax - t0) / TK + 1;

  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;
  const __bf16* kg = k + kv_base;
  const __bf16* vg = v + kv_base;

  const int tq = qfirst + lq;
  const bool row_ok = lq < nvalid;
  const size_t qrow = (size_t)(b * a.Hq + h) * a.S + tq;
  bf16x8 qreg[NKK], doreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (row_ok) {
      qreg[kk] = *reinterpret_cast<const bf16x8*>(q + qrow * D + 16 * kk + 8 * hi);
      doreg[kk] = *reinterpret_cast<const bf16x8*>(dO + qrow * D + 16 * kk + 8 * hi);
    } else {
      qreg[kk] = bf16x8{};
      doreg[kk] = bf16x8{};
    }
  }
  const float lse2 = row_ok ? lse[qrow] * kLog2e : 0.f;
  const float dlt = row_ok ? delta[(size_t)(b * a.Hq + h) * a.L + (tq - t0)] : 0.f;

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
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(&s_k[buf][(4 * rq + i) * KSTR + 8 * cc]) = kr[i];
      *reinterpret_cast<uint4*>(&s_v[buf][(4 * rq + i) * KSTR + 8 * cc]) = vr[i];
    }
    const int pos = tpos(4 * rq);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint2*>(&s_kt[buf][toff<TK>(8 * cc + e, pos)]) =
          quad_column(kr[0], kr[1], kr[2], kr[3], e);
  };

  floatx16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = floatx16{};

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
      const __bf16* vt = s_v[buf];
      const __bf16* ktt = s_kt[buf];
      floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        sacc = mfma32(lds_b128(kt + lq * KSTR + 16 * kk + 8 * hi), qreg[kk], sacc);
        pacc = mfma32(lds_b128(vt + lq * KSTR + 16 * kk + 8 * hi), doreg[kk], pacc);
      }
      const int hist_first = it * TK;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr_ = 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool ok = is_local ? (local_first + kr_ <= tq) : (hist_first + kr_ < src.nh);
        const float p = ok ? exp2f(sacc[r] * a.c2 - lse2) : 0.f;
        sacc[r] = p * (pacc[r] - dlt);  // dS^T
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int r0 = 8 * ks;
        const bf16x8 sb = to_bf16x8(sacc[r0], sacc[r0 + 1], sacc[r0 + 2], sacc[r0 + 3],
                                    sacc[r0 + 4], sacc[r0 + 5], sacc[r0 + 6], sacc[r0 + 7]);
        const int pos = 16 * ks + 8 * hi;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dqacc[db] = mfma32(lds_b128(ktt + toff<TK>(32 * db + lq, pos)), sb, dqacc[db]);
      }
    }
    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (active && row_ok) {
    __bf16* op = dq + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 pk;
        pk[0] = (__bf16)(dqacc[db][4 * r4 + 0] * a.scale);
        pk[1] = (__bf16)(dqacc[db][4 * r4 + 1] * a.scale);
        pk[2] = (__bf16)(dqacc[db][4 * r4 + 2] * a.scale);
        pk[3] = (__bf16)(dqacc[db][4 * r4 + 3] * a.scale);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * r4 + 4 * hi) = pk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// a8, bf16 MFMA: dk/dv of the local keys.  One block of threads per
// (b, g, 32-key tile kt of the segment); its 4 waves split the (query head,
// 32-query tile) pairs that see the key tile (query tiles kt.. of every
// head of the group) round-robin, each accumulating dK^T and dV^T for the
// 32 keys in registers; the 4 partial sums are folded through LDS at the
// end.  Per wave and pair (K and V rows of the tile in registers):
//   S  = Q . K^T   (Q rows straight from memory as A operand)
//   dP = dO . V^T  (dO rows likewise)
//   P  = exp2(S c2 - lse2), dS = P * (dP - delta)
//   dV^T += dO^T . P,  dK^T += Q^T . dS   (dO^T, Q^T staged transposed into
//                                          the wave's own LDS slice)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void dkdv_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ lse,
    const __bf16* __restrict__ dO, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, BwdArgs a) {
  constexpr int TQ = 32;                 // queries per tile
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int T_ELEMS = D * TQ;        // one transposed tile
  constexpr int RSTR = D + 4;            // fp32 fold row stride
  constexpr int LDS_STAGE = 4 * 2 * T_ELEMS * 2;        // bytes: 4 waves x (Qt, dOt)
  constexpr int LDS_FOLD = 4 * 32 * RSTR * 4;           // bytes: 4 waves x 32 keys x D fp32
  constexpr int LDS_BYTES = LDS_STAGE > LDS_FOLD ? LDS_STAGE : LDS_FOLD;
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[LDS_BYTES];

  const int nkt = (a.L + 31) / 32;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = w % nkt;
  const int g = (w / nkt) % a.Hkv;
  const int b = w / (nkt * a.Hkv);
  const int t0 = a.seg * a.L;
  const int tend = t0 + a.L;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lq = lane & 31, hi = lane >> 5;
  __bf16* s_qt = reinterpret_cast<__bf16*>(s_raw) + wave * 2 * T_ELEMS;
  __bf16* s_dot = s_qt + T_ELEMS;

  // K and V rows of this key tile as B operands: lane (key lq, hi) holds
  // K[key][16kk + 8hi .. +7]
  const int tk = t0 + kt * 32 + lq;
  const bool key_ok = tk < tend;
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S * D;
  bf16x8 kreg[NKK], vreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (key_ok) {
      kreg[kk] = *reinterpret_cast<const bf16x8*>(k + kv_base + (size_t)tk * D + 16 * kk + 8 * hi);
      vreg[kk] = *reinterpret_cast<const bf16x8*>(v + kv_base + (size_t)tk * D + 16 * kk + 8 * hi);
    } else {
      kreg[kk] = bf16x8{};
      vreg[kk] = bf16x8{};
    }
  }

  floatx16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkacc[db] = floatx16{}; dvacc[db] = floatx16{}; }

  const int nqt = (a.L + TQ - 1) / TQ;
  const int npairs = (nqt - kt) * a.G;
  for (int pi = wave; pi < npairs; pi += 4) {
    const int qt = kt + pi / a.G;
    const int hh = pi % a.G;
    const int h = g * a.G + hh;
    const int tq0 = t0 + qt * TQ;
    const size_t hrow = (size_t)(b * a.Hq + h) * a.S;

    // Q and dO rows as A operands: lane (row lq, hi)
    const bool qrow_ok = tq0 + lq < tend;
    bf16x8 qa[NKK], da[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (qrow_ok) {
        qa[kk] = *reinterpret_cast<const bf16x8*>(q + (hrow + tq0 + lq) * D + 16 * kk + 8 * hi);
        da[kk] = *reinterpret_cast<const bf16x8*>(dO + (hrow + tq0 + lq) * D + 16 * kk + 8 * hi);
      } else {
        qa[kk] = bf16x8{};
        da[kk] = bf16x8{};
      }
    }
    // lse2 and delta of the 16 query rows this lane holds in C layout
    float lse2[16], dl[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tqr = tq0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const bool ok = tqr < tend;
      lse2[r] = ok ? lse[hrow + tqr] * kLog2e : 0.f;
      dl[r] = ok ? delta[(size_t)(b * a.Hq + h) * a.L + (tqr - t0)] : 0.f;
    }
    // stage Q^T and dO^T into this wave's LDS slice: jobs of 4 rows x 8 dims
#pragma unroll
    for (int jb = lane; jb < (TQ / 4) * (D / 8); jb += 64) {
      const int rq = jb / (D / 8), cc = jb % (D / 8);
      uint4 x[4], y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tq0 + 4 * rq + i;
        if (t < tend) {
          x[i] = *reinterpret_cast<const uint4*>(q + (hrow + t) * D + 8 * cc);
          y[i] = *reinterpret_cast<const uint4*>(dO + (hrow + t) * D + 8 * cc);
        } else {
          x[i] = make_uint4(0, 0, 0, 0);
          y[i] = x[i];
        }
      }
      const int pos = tpos(4 * rq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        *reinterpret_cast<uint2*>(&s_qt[toff<TQ>(8 * cc + e, pos)]) =
            quad_column(x[0], x[1], x[2], x[3], e);
        *reinterpret_cast<uint2*>(&s_dot[toff<TQ>(8 * cc + e, pos)]) =
            quad_column(y[0], y[1], y[2], y[3], e);
      }
    }
    wave_lds_sync();

    floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      sacc = mfma32(qa[kk], kreg[kk], sacc);
      pacc = mfma32(da[kk], vreg[kk], pacc);
    }
    // C layout: lane = key lq, item r = query row 8(r/4)+4hi+(r%4) of the tile
    float pv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tqr = tq0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const bool ok = key_ok && tk <= tqr && tqr < tend;
      const float p = ok ? exp2f(sacc[r] * a.c2 - lse2[r]) : 0.f;
      pv[r] = p;
      sacc[r] = p * (pacc[r] - dl[r]);  // dS
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r0 = 8 * ks;
      const bf16x8 pb = to_bf16x8(pv[r0], pv[r0 + 1], pv[r0 + 2], pv[r0 + 3], pv[r0 + 4],
                                  pv[r0 + 5], pv[r0 + 6], pv[r0 + 7]);
      const bf16x8 sb = to_bf16x8(sacc[r0], sacc[r0 + 1], sacc[r0 + 2], sacc[r0 + 3],
                                  sacc[r0 + 4], sacc[r0 + 5], sacc[r0 + 6], sacc[r0 + 7]);
      const int pos = 16 * ks + 8 * hi;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvacc[db] = mfma32(lds_b128(s_dot + toff<TQ>(32 * db + lq, pos)), pb, dvacc[db]);
        dkacc[db] = mfma32(lds_b128(s_qt + toff<TQ>(32 * db + lq, pos)), sb, dkacc[db]);
      }
    }
    wave_lds_sync();
  }

  // fold the 4 waves' partial sums through LDS, then scale / round / store
  __syncthreads();
  float* fold = reinterpret_cast<float*>(s_raw);
  for (int pass = 0; pass < 2; ++pass) {
    const floatx16* acc = pass == 0 ? dkacc : dvacc;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 val = make_float4(acc[db][4 * r4], acc[db][4 * r4 + 1], acc[db][4 * r4 + 2],
                                 acc[db][4 * r4 + 3]);
        *reinterpret_cast<float4*>(&fold[(wave * 32 + lq) * RSTR + 32 * db + 8 * r4 + 4 * hi]) = val;
      }
    }
    __syncthreads();
    const float mul = pass == 0 ? a.scale : 1.f;
    __bf16* outp = pass == 0 ? dk : dv;
    constexpr int PER = D / 8;  // 8 threads per key row
    const int key = tid / 8, d0 = (tid % 8) * PER;
    const int tko = t0 + kt * 32 + key;
    if (tko < tend) {
#pragma unroll
      for (int e = 0; e < PER; e += 4) {
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float4 x = *reinterpret_cast<const float4*>(&fold[(ww * 32 + key) * RSTR + d0 + e]);
          s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
        }
        bf16x4 pk;
        pk[0] = (__bf16)(s.x * mul); pk[1] = (__bf16)(s.y * mul);
        pk[2] = (__bf16)(s.z * mul); pk[3] = (__bf16)(s.w * mul);
        *reinterpret_cast<bf16x4*>(outp + kv_base + (size_t)tko * D + d0 + e) = pk;
      }
    }
    __syncthreads();
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
    hipLaunchKernelGGL((dq_bf16_kernel<D>), dim3(nblocks), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, lse, (const __bf16*)dO, delta, sel,
                       (__bf16*)dq, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nblocks = p.B * p.Hkv * ((p.L + 31) / 32);
    ProfScope ps(HGA_K_BWD_DKDV, st);
    hipLaunchKernelGGL((dkdv_bf16_kernel<D>), dim3(nblocks), dim3(256), 0, st,
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
