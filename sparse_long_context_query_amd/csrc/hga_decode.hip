// Decode step of HGA for gfx950: attention of a few new tokens over the
// history blocks selected for them and the causal local part of their
// segment.
//
// [JA] 深掘り分析: after training, inference runs over sequences of up to
// 131,072 tokens while the resident block summaries grow; [JA] 業界への影響
// and [FR] Contexte: HGA as a module that speeds up retrieval and
// generation.  The pages give no decode procedure.  Reading: the n new
// tokens (positions pos .. pos+n-1, inside one segment starting at t0) form
// one query block of that segment: one selection per (sequence, KV head)
// from the mean of their queries over the G heads, then one joint softmax
// over the selected history tokens and the local tokens t0 .. pos+i.
//
// Work split (split over keys): per (sequence, KV head) the step's key list
// -- the selected history tokens in ascending order, then the local tokens
// t0 .. pos+n-1 -- is cut into chunks (64 keys; bf16 steps with more than
// 32 query rows: 128).  One block of 4 waves per (chunk, KV head, sequence)
// stages the chunk's K and V rows in LDS (every load in flight at once, each
// row read once) and writes the chunk's max, sum of exponentials and
// unnormalised P.V (fp32) for each of the R = G*n rows of the group to the
// workspace.  A merge kernel then combines the chunks of every row in chunk
// order (deterministic) into o and lse.  bf16 runs the chunk products on
// the matrix cores (decode_mfma_kernel: S^T = K.Q^T and O^T = V^T.P^T per
// 32-row tile of the G*n rows), f32 on the vector ALU (decode_attn_kernel,
// wave w taking the rows w, w+4, ...).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "hga_internal.h"
#include "hga_tiles.h"
#include "hga_topk.h"

namespace hga {
namespace {

constexpr int kCK = 64;     // keys per chunk (one per lane)
constexpr int kMaxRows = 64;  // G * n limit
// 64-key parts per chunk of decode_mfma_kernel: for up to 32 query rows
// (one row tile) and for more
constexpr int kPartsFewRows = 1;
constexpr int kPartsManyRows = 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecArgs {
  int S, Bh, Hq, Hkv, G, n, pos, t0, K;
  int nht;    // selected history tokens (k_eff * Bh)
  int nch_h;  // history chunks
  int nc;     // chunks in all
  float c2;   // softmax scale * log2(e)
  // bf16: the history chunks finish the top-k themselves from the m
  // candidates the scoring launch kept (ncs lists of K per (b, g))
  int fused, m, ncs;
  int ck;     // keys per chunk (kCK, or 128 for bf16 steps of over 32 rows)
};

template <typename T> struct Elt;
template <> struct Elt<__bf16> {
  __device__ __forceinline__ static float get(const __bf16* p, int i) { return (float)p[i]; }
};
template <> struct Elt<float> {
  __device__ __forceinline__ static float get(const float* p, int i) { return p[i]; }
};

// the wave's own LDS stores are visible to its later LDS loads
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// LDS layout of one wave (dynamic): q rows [R][D] f32, K rows [kCK][D + pad]
// (the 16-byte pad per row makes the lane-per-key reads conflict-free),
// V rows [kCK][D], then P [R][kCK] f32.
template <typename T, int D>
struct DecLds {
  static constexpr int EPP = 16 / sizeof(T);  // elements per 16-byte piece
  static constexpr int KP = D + EPP;          // K row pitch in elements
  static size_t bytes(int R) {
    return (size_t)R * D * 4 + (size_t)kCK * KP * sizeof(T) + (size_t)kCK * D * sizeof(T) +
           (size_t)R * kCK * 4;
  }
};

constexpr int kWaves = 4;  // waves per chunk block

template <typename T, int D>
__global__ __launch_bounds__(64 * kWaves) void decode_attn_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ sel, float* __restrict__ part_o, float* __restrict__ part_ml,
    DecArgs a) {
  using Lay = DecLds<T, D>;
  constexpr int EPP = Lay::EPP, KP = Lay::KP;
  constexpr int CPR = D / EPP;  // 16-byte pieces per row
  constexpr int ND = D / 64;    // output columns per lane
  extern __shared__ float4 dyn_lds[];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.G * a.n;
  float* qs = reinterpret_cast<float*>(dyn_lds);
  T* ks = reinterpret_cast<T*>(qs + (size_t)R * D);
  T* vs = ks + kCK * KP;
  float* ps = reinterpret_cast<float*>(vs + kCK * D);

  // token of key `key` of this chunk; rows that hold no key read a valid
  // row (masked below)
  auto token_of = [&](int key, bool& valid, bool& local) {
    if (c < a.nch_h) {
      const int hp = c * kCK + key;
      valid = hp < a.nht;
      local = false;
      return valid ? sel[(size_t)(b * a.Hkv + g) * a.K + hp / a.Bh] * a.Bh + hp % a.Bh : 0;
    }
    const int t = a.t0 + (c - a.nch_h) * kCK + key;
    valid = t < a.pos + a.n;
    local = true;
    return valid ? t : a.t0;
  };
  bool valid, local;
  const int tok = token_of(lane, valid, local);

  // stage K and V rows: thread tid moves pieces tid + 256 u of the chunk
  // (row = piece / CPR), all loads issued before the first LDS store
  constexpr int NPT = kCK * CPR / (64 * kWaves);  // pieces per thread
  const size_t kv_base = (size_t)(b * a.Hkv + g) * a.S;
  {
    uint4 kb[NPT], vb[NPT];
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int idx = tid + 64 * kWaves * u;
      const int r = idx / CPR, pc = idx % CPR;
      bool vr, lr;
      const int tr = token_of(r, vr, lr);
      const size_t src = (kv_base + tr) * D + pc * EPP;
      kb[u] = *reinterpret_cast<const uint4*>(k + src);
      vb[u] = *reinterpret_cast<const uint4*>(v + src);
    }
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int idx = tid + 64 * kWaves * u;
      const int r = idx / CPR, pc = idx % CPR;
      *reinterpret_cast<uint4*>(ks + r * KP + pc * EPP) = kb[u];
      *reinterpret_cast<uint4*>(vs + r * D + pc * EPP) = vb[u];
    }
  }
  for (int idx = tid; idx < R * D; idx += 64 * kWaves) {
    const int r = idx / D, d = idx % D;
    const int hh = r / a.n, i = r % a.n;
    qs[idx] = Elt<T>::get(q, (int)(((size_t)(b * a.Hq + g * a.G + hh) * a.n + i) * D + d));
  }
  __syncthreads();

  // scores in log2 units, one key per lane; then per row the chunk max,
  // exponentials and their sum
  float krow[D];
#pragma unroll
  for (int d = 0; d < D; ++d) krow[d] = Elt<T>::get(ks + lane * KP, d);
  float* ml = part_ml + ((size_t)(b * a.Hkv + g) * a.nc + c) * kMaxRows * 2;
  for (int r = wave; r < R; r += kWaves) {
    const float* qr = qs + (size_t)r * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const float4 q4 = *reinterpret_cast<const float4*>(qr + d);
      s += q4.x * krow[d] + q4.y * krow[d + 1] + q4.z * krow[d + 2] + q4.w * krow[d + 3];
    }
    const int i = r % a.n;
    const bool vis = valid && (!local || tok <= a.pos + i);
    const float z = vis ? s * a.c2 : -INFINITY;
    const float m = wave_max(z);
    const float p = vis ? exp2f(z - m) : 0.f;
    const float l = wave_sum(p);
    ps[r * kCK + lane] = p;
    if (lane == 0) {
      ml[2 * r] = m;
      ml[2 * r + 1] = l;
    }
  }
  wave_lds_fence();  // this wave's P rows, read back below by the same wave

  // unnormalised P.V: lane owns columns lane + 64 e
  float vcol[ND][kCK];
#pragma unroll
  for (int e = 0; e < ND; ++e)
#pragma unroll
    for (int kk = 0; kk < kCK; ++kk) vcol[e][kk] = Elt<T>::get(vs + kk * D, lane + 64 * e);
  float* po = part_o + ((size_t)(b * a.Hkv + g) * a.nc + c) * kMaxRows * D;
  for (int r = wave; r < R; r += kWaves) {
    float acc[ND];
#pragma unroll
    for (int e = 0; e < ND; ++e) acc[e] = 0.f;
    const float* pr = ps + r * kCK;
#pragma unroll
    for (int kk = 0; kk < kCK; kk += 4) {
      const float4 p4 = *reinterpret_cast<const float4*>(pr + kk);
#pragma unroll
      for (int e = 0; e < ND; ++e)
        acc[e] += p4.x * vcol[e][kk] + p4.y * vcol[e][kk + 1] + p4.z * vcol[e][kk + 2] +
                  p4.w * vcol[e][kk + 3];
    }
#pragma unroll
    for (int e = 0; e < ND; ++e) po[(size_t)r * D + lane + 64 * e] = acc[e];
  }
}

// Combines the chunks of query row r of (g, b) in chunk order, one wave
// (lane = column group).  With M = max_c m_c: l = sum_c l_c 2^(m_c - M),
// o = sum_c O_c 2^(m_c - M) / l, lse = (M + log2 l) ln 2.  The rows of the
// first kMergeBatch chunks do not depend on M and are requested together
// with the chunk maxima; later chunks follow in batches of as many.
constexpr int kMergeBatch = 16;

template <typename T, int D>
__device__ __forceinline__ void merge_row(const float* __restrict__ part_o,
                                          const float* __restrict__ part_ml, T* __restrict__ o,
                                          float* __restrict__ lse, const DecArgs& a, int r,
                                          int g, int b, int lane) {
  constexpr int ND = D / 64;
  constexpr int CB = kMergeBatch;
  const size_t base = (size_t)(b * a.Hkv + g) * a.nc;
  float x[CB][ND];
  auto request = [&](int c0) {
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int cc = min(c0 + u, a.nc - 1);
      const float* po = part_o + ((base + cc) * kMaxRows + r) * D;
#pragma unroll
      for (int e = 0; e < ND; ++e) x[u][e] = po[lane + 64 * e];
    }
  };
  request(0);
  // chunk maxima and sums, lane c holding chunk c (+ 64 j)
  float M = -INFINITY;
  float2 ml0 = make_float2(-INFINITY, 0.f);
  for (int c0 = 0; c0 < a.nc; c0 += 64) {
    const int c = c0 + lane;
    if (c < a.nc) {
      const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((base + c) * kMaxRows + r) * 2);
      if (c0 == 0) ml0 = ml;
      M = fmaxf(M, ml.x);
    }
  }
  M = wave_max(M);
  float l = 0.f, acc[ND];
#pragma unroll
  for (int e = 0; e < ND; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < a.nc; c0 += 64) {
    const int c = c0 + lane;
    float f = 0.f, lc = 0.f;
    if (c < a.nc) {
      const float2 ml =
          c0 == 0 ? ml0
                  : *reinterpret_cast<const float2*>(part_ml + ((base + c) * kMaxRows + r) * 2);
      // a chunk with no visible key of this row has ml = (-inf, 0)
      f = ml.y > 0.f ? exp2f(ml.x - M) : 0.f;
      lc = ml.y * f;
    }
    l += lc;
    const int cn = min(64, a.nc - c0);
    for (int j = 0; j < cn; j += CB) {
      if (c0 + j > 0) request(c0 + j);
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const float fj = __shfl(f, j + u, 64);
        if (j + u < cn)
#pragma unroll
          for (int e = 0; e < ND; ++e) acc[e] += x[u][e] * fj;
      }
    }
  }
  l = wave_sum(l);
  const int hh = r / a.n, i = r % a.n;
  const size_t orow = (size_t)(b * a.Hq + g * a.G + hh) * a.n + i;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < ND; ++e) o[orow * D + lane + 64 * e] = (T)(acc[e] * inv);
  if (lse != nullptr && lane == 0) lse[orow] = (M + log2f(l)) * kLn2;
}

// bf16, MFMA form of decode_attn_kernel (the same partial sums, over
// chunks of CK = 64 * 4 / RT keys).  The chunk's K and V rows are copied
// straight into swizzled row-major LDS tiles.  The R = G*n query rows (row r
// = head r / n, token r % n) form RT tiles of 32; wave w takes row tile
// w % RT and the 64 keys 64 (w / RT) .. +63 of the chunk, so all 4 waves
// work whatever n is, and, with Q^T in registers as the B operand:
//   S^T = K.Q^T (two 32-key halves),  per row: max m, P = exp2(S c2 - m) on
//   the visible keys, l = sum P,  O^T = V^T.P^T (V^T read transposed).
// The 4 / RT key parts of a row tile are then combined through LDS in part
// order (M = max m, l = sum l 2^(m - M), O likewise), and one wave writes
// the chunk's m, l and unnormalised O rows like decode_attn_kernel.  Larger
// chunks for fewer rows keep the partial sums the merge reads few.
// With a.fused, a history chunk first picks the k best of the m (score,
// index) candidates the scoring launch kept (each of its blocks' k best, in
// index order; wave_topk, the rule select_kernel applies, so every block
// finds the same set; chunk 0 also writes it to sel): the step then needs
// no top-k launch between the scores and the attention.
template <int D, int RT, int KPARTS>
__global__ __launch_bounds__(256) void decode_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    int32_t* __restrict__ sel, const float* __restrict__ cand_score,
    const int32_t* __restrict__ cand_idx, float* __restrict__ part_o,
    float* __restrict__ part_ml, DecArgs a) {
  static_assert(RT == 1 || RT == 2, "row tiles");
  static_assert(RT * KPARTS <= 4, "one wave per (row tile, key part)");
  // idle waves leave before the compute; the merge's barriers need all 4
  static_assert(KPARTS == 1 || RT * KPARTS == 4, "no idle wave with a merge");
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CK = 64 * KPARTS;       // keys per chunk (a.ck)
  constexpr int TILE_B = CK * 2 * D;
  constexpr int PART_B = 64 * 2 * D;    // bytes of one part's rows
  constexpr int CPR = (2 * D) / 16;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;         // rows per 1 KB copy instruction
  // the parts' O^T sums (64 lanes x NDB x 16 floats per wave) go where the
  // K rows were once every wave is done with them
  static_assert((KPARTS - 1) * RT * 64 * NDB * 16 * 4 <= TILE_B, "merge slots");
  __shared__ __attribute__((aligned(1024))) unsigned char s_k[TILE_B];
  __shared__ __attribute__((aligned(1024))) unsigned char s_v[TILE_B];
  __shared__ int s_sel[kMaxTopK];
  __shared__ float s_ml[4][32][2];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int bg = b * a.Hkv + g;
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.G * a.n;

  // the chosen history blocks: from sel, or (two-stage top-k) the k best of
  // the scoring launch's candidate lists, found here
  const int32_t* hsel = sel + (size_t)bg * a.K;
  if (a.fused && c < a.nch_h) {
    const float* cs = cand_score + (size_t)bg * a.ncs * a.K;
    const int32_t* ci = cand_idx + (size_t)bg * a.ncs * a.K;
    if (wave == 0) {  // the kept entries' block indices straight into s_sel
      if (a.m <= 64) wave_topk<1>(cs, a.m, a.K, s_sel, lane, ci);
      else if (a.m <= 128) wave_topk<2>(cs, a.m, a.K, s_sel, lane, ci);
      else if (a.m <= 256) wave_topk<4>(cs, a.m, a.K, s_sel, lane, ci);
      else if (a.m <= 512) wave_topk<8>(cs, a.m, a.K, s_sel, lane, ci);
      else wave_topk<16>(cs, a.m, a.K, s_sel, lane, ci);
    }
    __syncthreads();
    if (c == 0)
      for (int i = tid; i < a.K; i += 256) sel[(size_t)bg * a.K + i] = s_sel[i];
    hsel = s_sel;
  }

  // token of key `key` of this chunk; rows that hold no key read a valid row
  auto token_of = [&](int key, bool& valid, bool& local) {
    if (c < a.nch_h) {
      const int hp = c * CK + key;
      valid = hp < a.nht;
      local = false;
      return valid ? hsel[hp / a.Bh] * a.Bh + hp % a.Bh : 0;
    }
    const int t = a.t0 + (c - a.nch_h) * CK + key;
    valid = t < a.pos + a.n;
    local = true;
    return valid ? t : a.t0;
  };
  const size_t kv_base = (size_t)bg * a.S * D;
  {
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kv_base, (uint32_t)a.S * (2 * D));
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + kv_base, (uint32_t)a.S * (2 * D));
#pragma unroll
    for (int n = 0; n < CK / RPI / 4; ++n) {
      const int i = wave + 4 * n;
      const int row = i * RPI + lane / CPR;
      bool vld, loc;
      const int tok = token_of(row, vld, loc);
      const uint32_t off = (uint32_t)tok * (2 * D) + (((lane % CPR) ^ swz<D>(row)) << 4);
      buffer_to_lds16(kr, off, s_k + i * 1024);
      buffer_to_lds16(vr, off, s_v + i * 1024);
    }
  }
  // this wave's query rows as B operands: lane (row lq, hi) holds
  // Q[row][16kk + 8hi .. +7]
  const int rt = wave % RT, kp = wave / RT;
  const int r = 32 * rt + lq;
  const bool row_ok = r < R;
  const int hh = row_ok ? r / a.n : 0, ti = row_ok ? r % a.n : 0;
  bf16x8 qreg[NKK];
  {
    const __bf16* qp = q + ((size_t)(b * a.Hq + g * a.G + hh) * a.n + ti) * D + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qreg[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * kk) : bf16x8{};
  }
  drain_vmem_loads();
  __syncthreads();

  // waves past the RT * KPARTS (row tile, key part) pairs only copy
  if (wave >= RT * KPARTS) return;
  const unsigned char* sk = s_k + kp * PART_B;
  const unsigned char* sv = s_v + kp * PART_B;
  FragOffsets<D> fo;
  fo.init(lane);
  floatx16 sacc[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) sacc[st] = floatx16{};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int st = 0; st < 2; ++st) sacc[st] = mfma32(fo.row(sk, st, kk), qreg[kk], sacc[st]);
  // C layout: lane = query row lq, item rr of half st = key 32st + 8(rr/4) + 4hi + rr%4
  float mt = -INFINITY;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int key = 64 * kp + 32 * st + 8 * (rr >> 2) + 4 * hi + (rr & 3);
      // history keys: every selected token; local keys: up to this row's token
      const int tl = a.t0 + (c - a.nch_h) * CK + key;
      const bool vis = c < a.nch_h ? c * CK + key < a.nht : tl <= a.pos + ti;
      sacc[st][rr] = vis ? sacc[st][rr] * a.c2 : -INFINITY;
      mt = fmaxf(mt, sacc[st][rr]);
    }
  mt = pair_max(mt);
  float lsum = 0.f;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float p = mt == -INFINITY ? 0.f : exp2f(sacc[st][rr] - mt);
      sacc[st][rr] = p;
      lsum += p;
    }
  lsum = pair_sum(lsum);
  floatx16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = floatx16{};
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r0 = 8 * ks;
      const bf16x8 pb = to_bf16x8(sacc[st][r0], sacc[st][r0 + 1], sacc[st][r0 + 2],
                                  sacc[st][r0 + 3], sacc[st][r0 + 4], sacc[st][r0 + 5],
                                  sacc[st][r0 + 6], sacc[st][r0 + 7]);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32(fo.tr(sv, 32 * st + 16 * ks, db), pb, oacc[db]);
    }

  // combine the key parts of each row tile in part order: parts 1.. leave
  // (m, l) and O^T in LDS (the K rows' space, free once every wave is past
  // its score products), part 0 adds them
  if constexpr (KPARTS > 1) {
    float4* slots = reinterpret_cast<float4*>(s_k);
    __syncthreads();  // every wave is done reading the K rows
    if (kp > 0) {
      if (hi == 0) {
        s_ml[wave][lq][0] = mt;
        s_ml[wave][lq][1] = lsum;
      }
      float4* mine = slots + (size_t)(wave - RT) * NDB * 4 * 64 + lane;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          mine[(db * 4 + r4) * 64] = make_float4(oacc[db][4 * r4], oacc[db][4 * r4 + 1],
                                                 oacc[db][4 * r4 + 2], oacc[db][4 * r4 + 3]);
    }
    __syncthreads();
    if (kp > 0) return;
    float mp[KPARTS], lp[KPARTS];
    mp[0] = mt;
    lp[0] = lsum;
    float M = mt;
#pragma unroll
    for (int j = 1; j < KPARTS; ++j) {
      mp[j] = s_ml[rt + RT * j][lq][0];
      lp[j] = s_ml[rt + RT * j][lq][1];
      M = fmaxf(M, mp[j]);
    }
    // a part with no visible key of the row has (m, l) = (-inf, 0)
    float f[KPARTS];
    lsum = 0.f;
#pragma unroll
    for (int j = 0; j < KPARTS; ++j) {
      f[j] = lp[j] > 0.f ? exp2f(mp[j] - M) : 0.f;
      lsum += lp[j] * f[j];
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= f[0];
#pragma unroll
    for (int j = 1; j < KPARTS; ++j) {
      const float4* theirs = slots + (size_t)(rt + RT * j - RT) * NDB * 4 * 64 + lane;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 t = theirs[(db * 4 + r4) * 64];
          oacc[db][4 * r4] += t.x * f[j];
          oacc[db][4 * r4 + 1] += t.y * f[j];
          oacc[db][4 * r4 + 2] += t.z * f[j];
          oacc[db][4 * r4 + 3] += t.w * f[j];
        }
    }
    mt = M;
  }
  if (row_ok) {
    float* ml = part_ml + ((size_t)bg * a.nc + c) * kMaxRows * 2;
    if (hi == 0) {
      ml[2 * r] = mt;
      ml[2 * r + 1] = lsum;
    }
    float* po = part_o + (((size_t)bg * a.nc + c) * kMaxRows + r) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * r4 + 4 * hi) =
            make_float4(oacc[db][4 * r4], oacc[db][4 * r4 + 1], oacc[db][4 * r4 + 2],
                        oacc[db][4 * r4 + 3]);
  }
}

// One wave per (query row, KV head, sequence): merge_row.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, T* __restrict__ o,
    float* __restrict__ lse, DecArgs a) {
  merge_row<T, D>(part_o, part_ml, o, lse, a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x);
}

struct DecPlan {
  DecArgs a;
  int R;
};

DecPlan plan(const Prob& p, int pos, int n) {
  DecPlan d;
  DecArgs& a = d.a;
  a.S = p.S;
  a.Bh = p.Bh;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.n = n;
  a.pos = pos;
  a.t0 = pos / p.L * p.L;
  a.K = p.K;
  const int nb = a.t0 / p.Bh;
  // bf16: decode_mfma_kernel's chunks, 64 keys per part
  a.ck = p.dtype == HGA_BF16 ? 64 * (p.G * n <= 32 ? kPartsFewRows : kPartsManyRows) : kCK;
  a.nht = (nb < p.K ? nb : p.K) * p.Bh;
  a.nch_h = (a.nht + a.ck - 1) / a.ck;
  a.nc = a.nch_h + (pos + n - a.t0 + a.ck - 1) / a.ck;
  a.c2 = p.scale * kLog2e;
  a.fused = 0;
  a.ncs = decode_cand_slots(p);
  const int cpb = decode_scoring_block(p, nb);
  a.m = (nb + cpb - 1) / cpb * p.K;
  d.R = p.G * n;
  return d;
}

int max_chunks(const Prob& p) {
  const int nb_max = (p.S - p.L) / p.Bh;  // history blocks of the last segment
  const int nht = (nb_max < p.K ? nb_max : p.K) * p.Bh;
  return (nht + kCK - 1) / kCK + (p.L + kCK - 1) / kCK;
}

template <typename T, int D>
hipError_t decode_t(const Prob& p, int pos, int n, const void* q_new, const void* k,
                    const void* v, int32_t* sel, void* o, float* lse, float* ws, bool fused,
                    hipStream_t st) {
  DecPlan d = plan(p, pos, n);
  float* part_o = ws;
  float* part_ml = ws + (size_t)p.B * p.Hkv * max_chunks(p) * kMaxRows * p.D;
  if constexpr (std::is_same<T, __bf16>::value) {
    d.a.fused = fused ? 1 : 0;
    if (d.R <= 32)
      HGA_LAUNCH(HGA_K_DECODE, (decode_mfma_kernel<D, 1, kPartsFewRows>), dim3(d.a.nc, p.Hkv, p.B),
                 dim3(256), 0, st, (const __bf16*)q_new, (const __bf16*)k, (const __bf16*)v, sel,
                 (const float*)decode_cand_score_ws(p, ws),
                 (const int32_t*)decode_cand_idx_ws(p, ws), part_o, part_ml, d.a);
    else
      HGA_LAUNCH(HGA_K_DECODE, (decode_mfma_kernel<D, 2, kPartsManyRows>), dim3(d.a.nc, p.Hkv, p.B),
                 dim3(256), 0, st, (const __bf16*)q_new, (const __bf16*)k, (const __bf16*)v, sel,
                 (const float*)decode_cand_score_ws(p, ws),
                 (const int32_t*)decode_cand_idx_ws(p, ws), part_o, part_ml, d.a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    HGA_LAUNCH(HGA_K_DECODE_MERGE, (decode_merge_kernel<T, D>), dim3(d.R, p.Hkv, p.B), dim3(64),
               0, st, (const float*)part_o, (const float*)part_ml, (T*)o, lse, d.a);
    return hipGetLastError();
  }
  const size_t shm = DecLds<T, D>::bytes(d.R);
  if (shm > 32768) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_attn_kernel<T, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  {
    HGA_LAUNCH(HGA_K_DECODE, (decode_attn_kernel<T, D>), dim3(d.a.nc, p.Hkv, p.B), dim3(64 * kWaves),
                       shm, st,
                       (const T*)q_new, (const T*)k, (const T*)v, sel, part_o, part_ml, d.a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  HGA_LAUNCH(HGA_K_DECODE_MERGE, (decode_merge_kernel<T, D>), dim3(d.R, p.Hkv, p.B), dim3(64), 0, st,
             
                     (const float*)part_o, (const float*)part_ml, (T*)o, lse, d.a);
  return hipGetLastError();
}

}  // namespace

int decode_max_rows() { return kMaxRows; }

// Workspace: chunk partial O [B, Hkv, chunks, 64, D], then the chunk (max,
// sum) pairs [B, Hkv, chunks, 64, 2], then the selection scores
// [B, Hkv, nblk], all float32; then the two-stage top-k's candidate scores
// [B, Hkv, slots, k] float32 and block indices [B, Hkv, slots, k] int32.
static size_t partial_floats(const Prob& p) {
  return (size_t)p.B * p.Hkv * max_chunks(p) * kMaxRows * (p.D + 2);
}

int decode_cand_slots(const Prob& p) { return (std::min(p.nblk, 1024) + 127) / 128; }

int decode_scoring_block(const Prob& p, int nb) { return (nb + 127) / 128 * p.K <= 1024 ? 128 : 256; }

static size_t cand_entries(const Prob& p) {
  return (size_t)p.B * p.Hkv * decode_cand_slots(p) * p.K;
}

size_t decode_workspace_bytes(const Prob& p) {
  return (partial_floats(p) + (size_t)p.B * p.Hkv * p.nblk + cand_entries(p)) * sizeof(float) +
         cand_entries(p) * sizeof(int32_t);
}

float* decode_score_ws(const Prob& p, void* ws) {
  return reinterpret_cast<float*>(ws) + partial_floats(p);
}

float* decode_cand_score_ws(const Prob& p, void* ws) {
  return decode_score_ws(p, ws) + (size_t)p.B * p.Hkv * p.nblk;
}

int32_t* decode_cand_idx_ws(const Prob& p, void* ws) {
  return reinterpret_cast<int32_t*>(decode_cand_score_ws(p, ws) + cand_entries(p));
}

// two-stage top-k: k < nb <= 1,024 history blocks, k <= 256 (one block's
// list), and at most 1,024 candidates left for the attention blocks' search
// (with 256-candidate scoring blocks at the most)
bool decode_fused(const Prob& p, int pos, int n) {
  (void)n;
  const int nb = pos / p.L * p.L / p.Bh;
  return p.dtype == HGA_BF16 && nb > p.K && nb <= 1024 && p.K <= 256 &&
         (nb + 255) / 256 * p.K <= 1024;
}

hipError_t launch_decode(const Prob& p, int pos, int n, const void* q_new, const void* k,
                         const void* v, int32_t* sel, void* o, float* lse, float* ws, bool fused,
                         hipStream_t st) {
  if (p.dtype == HGA_BF16)
    return p.D == 64
               ? decode_t<__bf16, 64>(p, pos, n, q_new, k, v, sel, o, lse, ws, fused, st)
               : decode_t<__bf16, 128>(p, pos, n, q_new, k, v, sel, o, lse, ws, fused, st);
  return p.D == 64 ? decode_t<float, 64>(p, pos, n, q_new, k, v, sel, o, lse, ws, false, st)
                   : decode_t<float, 128>(p, pos, n, q_new, k, v, sel, o, lse, ws, false, st);
}

}  // namespace hga
