// C ABI of the HGA hot path: host-side validation, dispatch and the
// optional per-kernel profiling hooks.  Every argument check happens here,
// before anything is enqueued; no C++ exception leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "hga.h"
#include "hga_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return HGA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HGA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Builds the derived problem description, or returns an error code.
int make_prob(const hga_config* c, hga::Prob* p) {
  if (c == nullptr) return fail(HGA_ERR_ARG, "config is NULL");
  if (c->batch < 1 || c->seq_len < 1 || c->seg_len < 1 || c->hist_block < 1 ||
      c->query_block < 1 || c->top_k < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 1)
    return fail(HGA_ERR_ARG, "every size in the config must be >= 1");
  if (c->seq_len % c->seg_len)
    return fail(HGA_ERR_ARG, "seq_len %d is not a multiple of seg_len %d", c->seq_len, c->seg_len);
  if (c->seg_len % c->hist_block)
    return fail(HGA_ERR_ARG, "seg_len %d is not a multiple of hist_block %d", c->seg_len,
                c->hist_block);
  if (c->seg_len % c->query_block)
    return fail(HGA_ERR_ARG, "seg_len %d is not a multiple of query_block %d", c->seg_len,
                c->query_block);
  if (c->n_q_heads % c->n_kv_heads)
    return fail(HGA_ERR_ARG, "n_q_heads %d is not a multiple of n_kv_heads %d", c->n_q_heads,
                c->n_kv_heads);
  if (c->dtype != HGA_F32 && c->dtype != HGA_BF16)
    return fail(HGA_ERR_UNSUPPORTED, "dtype %d is not supported (F32=0, BF16=1)", c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(HGA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", c->head_dim);
  if (c->seq_len / c->hist_block > hga::kMaxCandidates)
    return fail(HGA_ERR_UNSUPPORTED, "seq_len/hist_block = %d exceeds %d history blocks",
                c->seq_len / c->hist_block, hga::kMaxCandidates);
  if (c->top_k > hga::kMaxTopK)
    return fail(HGA_ERR_UNSUPPORTED, "top_k %d exceeds %d", c->top_k, hga::kMaxTopK);
  if (c->dtype == HGA_BF16 && (c->hist_block % 16 || c->query_block % 16))
    return fail(HGA_ERR_UNSUPPORTED,
                "bf16 kernels need hist_block and query_block to be multiples of 16");
  if (c->dtype == HGA_F32 && c->hist_block % 4)
    return fail(HGA_ERR_UNSUPPORTED, "f32 kernels need hist_block to be a multiple of 4");
  // the bf16 kernels address one (sequence, head) slice of a tensor through a
  // buffer resource with a 32-bit byte count
  if ((double)c->seq_len * c->head_dim * (c->dtype == HGA_F32 ? 4 : 2) > 2147483647.0)
    return fail(HGA_ERR_UNSUPPORTED, "seq_len*head_dim of one head exceeds 2 GiB");
  const double elems = (double)c->batch * c->n_q_heads * c->seq_len * c->head_dim;
  if (elems > 2147483647.0 * 64)
    return fail(HGA_ERR_UNSUPPORTED, "tensor too large");
  if (!(std::isfinite(c->softmax_scale)))
    return fail(HGA_ERR_ARG, "softmax_scale is not finite");
  p->B = c->batch;
  p->S = c->seq_len;
  p->L = c->seg_len;
  p->Bh = c->hist_block;
  p->Bq = c->query_block;
  p->K = c->top_k;
  p->Hq = c->n_q_heads;
  p->Hkv = c->n_kv_heads;
  p->D = c->head_dim;
  p->G = c->n_q_heads / c->n_kv_heads;
  p->dtype = c->dtype;
  p->scale = c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / std::sqrt((float)c->head_dim);
  p->nqb = p->L / p->Bq;
  p->nqb_all = p->S / p->Bq;
  p->nblk = p->S / p->Bh;
  p->kv_rows = p->S;
  p->kv_local = -1;
  return HGA_OK;
}

int check_seg(const hga::Prob& p, int32_t seg) {
  if (seg < 0 || seg >= p.S / p.L)
    return fail(HGA_ERR_ARG, "segment %d out of range [0, %d)", seg, p.S / p.L);
  return HGA_OK;
}

#define HGA_REQUIRE(ptr)                                              \
  do {                                                                \
    if ((ptr) == nullptr) return fail(HGA_ERR_ARG, #ptr " is NULL");  \
  } while (0)

// ---- profiling -----------------------------------------------------------
struct ProfEvent {
  int kclass;
  hipEvent_t start, stop;
};
thread_local bool g_prof_on = false;
thread_local uint32_t g_prof_mask = 0;
thread_local std::vector<ProfEvent> g_prof_events;
thread_local std::vector<hipEvent_t> g_prof_pool;

hipEvent_t pool_get() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace hga {
bool prof_events(int kclass, hipEvent_t* start, hipEvent_t* stop) {
  if (!g_prof_on || !((g_prof_mask >> kclass) & 1u)) return false;
  hipEvent_t a = pool_get();
  hipEvent_t b = a ? pool_get() : nullptr;
  if (b == nullptr) {
    if (a) g_prof_pool.push_back(a);
    return false;
  }
  g_prof_events.push_back({kclass, a, b});
  *start = a;
  *stop = b;
  return true;
}
}  // namespace hga

namespace {

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace of hga_segment_pass.  bf16: the delta rows of every segment
// (written by the forward launch, read by the backward launches).  f32: one
// step workspace per stream.
size_t pass_exact_workspace_bytes(const hga::Prob& p);
size_t tier_workspace_bytes(const hga::Prob& p, int nwin);
int check_tier(const hga::Prob& p);

size_t pass_workspace_bytes(const hga::Prob& p) {
  if (p.dtype == HGA_BF16) return (size_t)(p.S / p.L) * hga::bwd_delta_bytes(p);
  return 2 * round256(hga::bwd_workspace_bytes(p));
}

// Workspace of hga_segment_pass_exact: every segment's delta rows, the fp32
// history sums of dK and dV ([B, Hkv, S, D] each), every segment's history
// block list.
size_t pass_exact_workspace_bytes(const hga::Prob& p) {
  const size_t sums = round256((size_t)p.B * p.Hkv * p.S * p.D * sizeof(float));
  return (size_t)(p.S / p.L) * hga::bwd_delta_bytes(p) + 2 * sums + hga::hist_lists_bytes(p);
}

}  // namespace

extern "C" {

const char* hga_last_error(void) { return g_last_error.c_str(); }

const char* hga_version(void) { return "hga-mi355x 0.1 (gfx950)"; }

size_t hga_workspace_size(const hga_config* cfg, int32_t op) {
  hga::Prob p;
  if (make_prob(cfg, &p) != HGA_OK) return 0;
  switch (op) {
    case HGA_OP_FWD:
      ok();
      return 0;
    case HGA_OP_BWD:
    case HGA_OP_STEP:
      ok();
      return hga::bwd_workspace_bytes(p);
    case HGA_OP_DECODE:
      ok();
      return hga::decode_workspace_bytes(p);
    case HGA_OP_STEP_EXACT:
      ok();
      return hga::bwd_exact_workspace_bytes(p);
    case HGA_OP_PASS:
      ok();
      return pass_workspace_bytes(p);
    case HGA_OP_PASS_EXACT:
      ok();
      return pass_exact_workspace_bytes(p);
    case HGA_OP_STEP_HOST:
    case HGA_OP_PASS_HOST:
      if (check_tier(p)) return 0;
      ok();
      return tier_workspace_bytes(p, op == HGA_OP_STEP_HOST ? 1 : 2);
    default:
      fail(HGA_ERR_ARG, "unknown op %d", op);
      return 0;
  }
}

int hga_summarize(const hga_config* cfg, const void* k, int32_t blk_begin, int32_t blk_end,
                  float* summ, void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  HGA_REQUIRE(k);
  HGA_REQUIRE(summ);
  if (blk_begin < 0 || blk_end < blk_begin || blk_end > p.nblk)
    return fail(HGA_ERR_ARG, "block range [%d, %d) outside [0, %d]", blk_begin, blk_end, p.nblk);
  hipError_t e = hga::launch_summarize(p, k, blk_begin, blk_end, summ, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "summarize launch");
  return ok();
}

int hga_select(const hga_config* cfg, const void* q, const float* summ, int32_t seg,
               int32_t* sel, void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if ((rc = check_seg(p, seg))) return rc;
  HGA_REQUIRE(q);
  HGA_REQUIRE(summ);
  HGA_REQUIRE(sel);
  hipError_t e = hga::launch_select(p, q, summ, seg, sel, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

int hga_gather(const hga_config* cfg, const void* k, const void* v, const int32_t* sel,
               int32_t seg, void* k_out, void* v_out, void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if ((rc = check_seg(p, seg))) return rc;
  HGA_REQUIRE(k);
  HGA_REQUIRE(v);
  HGA_REQUIRE(sel);
  HGA_REQUIRE(k_out);
  HGA_REQUIRE(v_out);
  hipError_t e = hga::launch_gather(p, k, v, sel, seg, k_out, v_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

int hga_attn_fwd(const hga_config* cfg, const void* q, const void* k, const void* v,
                 const int32_t* sel, int32_t seg, void* o, float* lse, void* ws,
                 size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if ((rc = check_seg(p, seg))) return rc;
  HGA_REQUIRE(q);
  HGA_REQUIRE(k);
  HGA_REQUIRE(v);
  HGA_REQUIRE(sel);
  HGA_REQUIRE(o);
  hipError_t e = hga::launch_fwd(p, q, k, v, sel, seg, o, lse, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

int hga_attn_bwd(const hga_config* cfg, const void* q, const void* k, const void* v,
                 const void* o, const float* lse, const void* dO, const int32_t* sel,
                 int32_t seg, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                 void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if ((rc = check_seg(p, seg))) return rc;
  HGA_REQUIRE(q);
  HGA_REQUIRE(k);
  HGA_REQUIRE(v);
  HGA_REQUIRE(o);
  HGA_REQUIRE(lse);
  HGA_REQUIRE(dO);
  HGA_REQUIRE(sel);
  HGA_REQUIRE(dq);
  HGA_REQUIRE(dk);
  HGA_REQUIRE(dv);
  HGA_REQUIRE(ws);
  const size_t need = hga::bwd_workspace_bytes(p);
  if (ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  hipError_t e = hga::launch_bwd(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, (float*)ws,
                                 (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

}  // extern "C"

namespace {

// Argument checks shared by the step and the pass (everything but seg).
int check_step_args(const hga::Prob& p, int32_t flags, const void* q, const void* k,
                    const void* v, const void* dO, const float* summ, const int32_t* sel,
                    const void* o, const float* lse, const void* dq, const void* dk,
                    const void* dv, const void* ws, size_t ws_bytes, size_t ws_need) {
  if (flags & ~(HGA_STEP_BWD | HGA_STEP_SUMMARIES_READY))
    return fail(HGA_ERR_ARG, "unknown flags 0x%x", flags);
  HGA_REQUIRE(q);
  HGA_REQUIRE(k);
  HGA_REQUIRE(v);
  HGA_REQUIRE(summ);
  HGA_REQUIRE(sel);
  HGA_REQUIRE(o);
  if (flags & HGA_STEP_BWD) {
    HGA_REQUIRE(lse);
    HGA_REQUIRE(dO);
    HGA_REQUIRE(dq);
    HGA_REQUIRE(dk);
    HGA_REQUIRE(dv);
    HGA_REQUIRE(ws);
    if (ws_bytes < ws_need)
      return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  ws_bytes, ws_need);
  }
  (void)p;
  return HGA_OK;
}

// One validated segment step on stream st.
int run_step(const hga::Prob& p, int32_t seg, int32_t flags, const void* q, const void* k,
             const void* v, const void* dO, float* summ, int32_t* sel, void* o, float* lse,
             void* dq, void* dk, void* dv, void* ws, hipStream_t st) {
  const bool bwd = (flags & HGA_STEP_BWD) != 0;
  hipError_t e;
  if (seg > 0 && !(flags & HGA_STEP_SUMMARIES_READY)) {
    // blocks closed by segment seg-1 become history of segment seg
    const int b0 = (seg - 1) * p.L / p.Bh, b1 = seg * p.L / p.Bh;
    e = hga::launch_summarize(p, k, b0, b1, summ, st);
    if (e != hipSuccess) return hip_fail(e, "summarize launch");
  }
  e = hga::launch_select(p, q, summ, seg, sel, st);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  // with the backward to follow, the forward also writes its row sums
  // delta = rowsum(dO * o) into the workspace (bf16), saving the backward a pass
  const bool fuse = bwd && hga::fused_delta(p);
  e = hga::launch_fwd(p, q, k, v, sel, seg, o, lse, st, fuse ? dO : nullptr,
                      fuse ? (float*)ws : nullptr);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  if (bwd) {
    e = hga::launch_bwd(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, (float*)ws, st, fuse);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
  }
  return HGA_OK;
}

// Stream hand-off events of the passes, per calling thread and per device
// (an event belongs to the device that was current when it was made):
// [0, 2) the f32 pass's, [2, 7) the host-tier pass's.  Created on first use
// and kept; timing disabled, they only order work.
constexpr int kMaxDevices = 64;
constexpr int kPassEvents = 7;
hipError_t device_events(hipEvent_t** out) {
  thread_local hipEvent_t ev[kMaxDevices][kPassEvents] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  for (int i = 0; i < kPassEvents; ++i)
    if (ev[dev][i] == nullptr &&
        (e = hipEventCreateWithFlags(&ev[dev][i], hipEventDisableTiming)) != hipSuccess)
      return e;
  *out = ev[dev];
  return hipSuccess;
}

// Scratch array of hga_segment_pass_noalloc, one per GPU (each device holds
// its own copy from the code object's load until the process ends).  In
// host code `scratch` is only a handle for hipGetSymbolAddress: host code
// passes the device address scratch_address() returns, never the name.
constexpr size_t kNoallocScratchBytes = HGA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t pass_events(hipEvent_t* a, hipEvent_t* b) {
  hipEvent_t* ev = nullptr;
  const hipError_t e = device_events(&ev);
  if (e != hipSuccess) return e;
  *a = ev[0];
  *b = ev[1];
  return hipSuccess;
}

// ---- host-RAM history tier -------------------------------------------------
// Workspace: the backward's scratch, the selection in window slots (wsel,
// the layout of sel), then one or two windows, each the K and V rows
// [B, Hkv, C*Bh + L, D] (C = tier_slots), the slot list [B, Hkv, C] and the
// union sizes [B, Hkv].
struct TierWs {
  void* bws;
  int32_t* wsel;
  void* kw[2];
  void* vw[2];
  int32_t* list[2];
  int32_t* count[2];
};

size_t tier_kv_bytes(const hga::Prob& p) {
  return round256((size_t)p.B * p.Hkv * hga::tier_rows(p) * p.D * 2);
}
size_t tier_list_bytes(const hga::Prob& p) {
  return round256((size_t)p.B * p.Hkv * std::max(hga::tier_slots(p), 1) * sizeof(int32_t));
}
size_t tier_count_bytes(const hga::Prob& p) {
  return round256((size_t)p.B * p.Hkv * sizeof(int32_t));
}
size_t tier_wsel_bytes(const hga::Prob& p) {
  return round256((size_t)p.B * p.Hkv * p.nqb_all * p.K * sizeof(int32_t));
}
size_t tier_workspace_bytes(const hga::Prob& p, int nwin) {
  const size_t win = 2 * tier_kv_bytes(p) + tier_list_bytes(p) + tier_count_bytes(p);
  return round256(hga::bwd_workspace_bytes(p)) + tier_wsel_bytes(p) + nwin * win;
}
TierWs tier_carve(const hga::Prob& p, void* ws, int nwin) {
  TierWs t;
  char* c = (char*)ws;
  t.bws = c;
  c += round256(hga::bwd_workspace_bytes(p));
  t.wsel = (int32_t*)c;
  c += tier_wsel_bytes(p);
  for (int w = 0; w < 2; ++w) {
    if (w < nwin) {
      t.kw[w] = c; c += tier_kv_bytes(p);
      t.vw[w] = c; c += tier_kv_bytes(p);
      t.list[w] = (int32_t*)c; c += tier_list_bytes(p);
      t.count[w] = (int32_t*)c; c += tier_count_bytes(p);
    } else {
      t.kw[w] = t.kw[0]; t.vw[w] = t.vw[0]; t.list[w] = t.list[0]; t.count[w] = t.count[0];
    }
  }
  return t;
}

// The device address of pinned host memory (the kernels read it directly).
int host_pointer(const void* h, const char* name, const void** dptr) {
  hipPointerAttribute_t at;
  const hipError_t e = hipPointerGetAttributes(&at, h);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(HGA_ERR_ARG, "%s is not pinned host memory (%s)", name, hipGetErrorString(e));
  }
  if (at.type != hipMemoryTypeHost || at.devicePointer == nullptr)
    return fail(HGA_ERR_ARG, "%s is not pinned host memory", name);
  *dptr = at.devicePointer;
  return HGA_OK;
}

int check_tier(const hga::Prob& p) {
  if (p.dtype != HGA_BF16)
    return fail(HGA_ERR_UNSUPPORTED, "the host tier runs the bf16 kernels only");
  return HGA_OK;
}

// The window's geometry for the step kernels.
hga::Prob tier_prob(const hga::Prob& p) {
  hga::Prob pw = p;
  pw.kv_rows = hga::tier_rows(p);
  pw.kv_local = hga::tier_slots(p) * p.Bh;
  return pw;
}

// The summaries of segment seg's own blocks (history of the later segments),
// read from window w, where the fetch put the segment's rows.  The last
// segment's blocks are never history.
int tier_summarize(const hga::Prob& p, int32_t seg, float* summ, const TierWs& t, int w,
                   hipStream_t st) {
  if (seg + 1 >= p.S / p.L) return HGA_OK;
  const hga::Prob pw = tier_prob(p);
  const hipError_t e = hga::launch_summarize(pw, t.kw[w], seg * p.L / p.Bh,
                                             (seg + 1) * p.L / p.Bh, summ, st,
                                             pw.kv_local - seg * p.L);
  return e == hipSuccess ? HGA_OK : hip_fail(e, "summarize launch");
}

// The selection of segment seg and the plan of window w's fetch, on st.
int tier_plan_step(const hga::Prob& p, int32_t seg, const void* q, const float* summ,
                   int32_t* sel, const TierWs& t, int w, hipStream_t st) {
  hipError_t e = hga::launch_select(p, q, summ, seg, sel, st);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  e = hga::launch_tier_plan(p, sel, seg, t.wsel, t.list[w], t.count[w], st);
  if (e != hipSuccess) return hip_fail(e, "tier plan launch");
  return HGA_OK;
}

// The selection of segment seg, then the fetch of what it chose, on st.
int tier_fetch_step(const hga::Prob& p, int32_t seg, const void* q, const void* kh,
                    const void* vh, const float* summ, int32_t* sel, const TierWs& t, int w,
                    hipStream_t st) {
  int rc = tier_plan_step(p, seg, q, summ, sel, t, w, st);
  if (rc) return rc;
  const hipError_t e =
      hga::launch_tier_fetch(p, kh, vh, t.list[w], t.count[w], seg, t.kw[w], t.vw[w], st);
  return e == hipSuccess ? HGA_OK : hip_fail(e, "tier fetch launch");
}

// The attention of segment seg over window w, on st.
int tier_attn_step(const hga::Prob& p, int32_t seg, bool bwd, const void* q, const void* dO,
                   void* o, float* lse, void* dq, void* dk, void* dv, const TierWs& t, int w,
                   hipStream_t st) {
  const hga::Prob pw = tier_prob(p);
  hipError_t e = hga::launch_fwd(pw, q, t.kw[w], t.vw[w], t.wsel, seg, o, lse, st,
                                 bwd ? dO : nullptr, bwd ? (float*)t.bws : nullptr);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  if (bwd) {
    e = hga::launch_bwd(pw, q, t.kw[w], t.vw[w], o, lse, dO, t.wsel, seg, dq, dk, dv,
                        (float*)t.bws, st, true);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
  }
  return HGA_OK;
}

// Events for the host-tier pass: [0, 2) fetch of window w done, [2, 4)
// attention over window w done, [4] inputs ready.
hipError_t tier_events(hipEvent_t** out) {
  hipEvent_t* ev = nullptr;
  const hipError_t e = device_events(&ev);
  if (e != hipSuccess) return e;
  *out = ev + 2;
  return hipSuccess;
}

}  // namespace

extern "C" {

int hga_segment_step(const hga_config* cfg, int32_t seg, int32_t flags, const void* q,
                     const void* k, const void* v, const void* dO, float* summ, int32_t* sel,
                     void* o, float* lse, void* dq, void* dk, void* dv, void* ws,
                     size_t ws_bytes, void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if ((rc = check_seg(p, seg))) return rc;
  if ((rc = check_step_args(p, flags, q, k, v, dO, summ, sel, o, lse, dq, dk, dv, ws, ws_bytes,
                            hga::bwd_workspace_bytes(p))))
    return rc;
  if ((rc = run_step(p, seg, flags, q, k, v, dO, summ, sel, o, lse, dq, dk, dv, ws,
                     (hipStream_t)stream)))
    return rc;
  return ok();
}

int hga_segment_step_host(const hga_config* cfg, int32_t seg, int32_t flags, const void* q,
                          const void* k_host, const void* v_host, const void* dO, float* summ,
                          int32_t* sel, void* o, float* lse, void* dq, void* dk, void* dv,
                          void* ws, size_t ws_bytes, void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if ((rc = check_tier(p))) return rc;
  if ((rc = check_seg(p, seg))) return rc;
  const size_t need = tier_workspace_bytes(p, 1);
  if ((rc = check_step_args(p, flags, q, k_host, v_host, dO, summ, sel, o, lse, dq, dk, dv, ws,
                            ws_bytes, need)))
    return rc;
  HGA_REQUIRE(ws);
  if (ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  const void *kh, *vh;
  if ((rc = host_pointer(k_host, "k_host", &kh))) return rc;
  if ((rc = host_pointer(v_host, "v_host", &vh))) return rc;
  const TierWs t = tier_carve(p, ws, 1);
  hipStream_t st = (hipStream_t)stream;
  if ((rc = tier_fetch_step(p, seg, q, kh, vh, summ, sel, t, 0, st))) return rc;
  if (!(flags & HGA_STEP_SUMMARIES_READY) && (rc = tier_summarize(p, seg, summ, t, 0, st)))
    return rc;
  if ((rc = tier_attn_step(p, seg, (flags & HGA_STEP_BWD) != 0, q, dO, o, lse, dq, dk, dv, t, 0,
                           st)))
    return rc;
  return ok();
}

int hga_segment_pass_host(const hga_config* cfg, int32_t flags, const void* q,
                          const void* k_host, const void* v_host, const void* dO, float* summ,
                          int32_t* sel, void* o, float* lse, void* dq, void* dk, void* dv,
                          void* ws, size_t ws_bytes, void* stream, void* stream2) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if ((rc = check_tier(p))) return rc;
  if (flags & HGA_STEP_SUMMARIES_READY)
    return fail(HGA_ERR_ARG, "the pass summarizes the history itself");
  const size_t need = tier_workspace_bytes(p, 2);
  if ((rc = check_step_args(p, flags, q, k_host, v_host, dO, summ, sel, o, lse, dq, dk, dv, ws,
                            ws_bytes, need)))
    return rc;
  HGA_REQUIRE(ws);
  if (ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  const void *kh, *vh;
  if ((rc = host_pointer(k_host, "k_host", &kh))) return rc;
  if ((rc = host_pointer(v_host, "v_host", &vh))) return rc;
  const TierWs t = tier_carve(p, ws, 2);
  const bool bwd = (flags & HGA_STEP_BWD) != 0;
  // attention on stream, the next segment's selection and fetch on stream2
  hipStream_t sa = (hipStream_t)stream;
  hipStream_t sf = stream2 != nullptr ? (hipStream_t)stream2 : sa;
  const bool two = sf != sa;
  hipEvent_t* ev = nullptr;
  hipError_t e;
  if (two) {
    if ((e = tier_events(&ev)) != hipSuccess) return hip_fail(e, "event create");
    if ((e = hipEventRecord(ev[4], sa)) != hipSuccess) return hip_fail(e, "event record");
    if ((e = hipStreamWaitEvent(sf, ev[4], 0)) != hipSuccess) return hip_fail(e, "stream wait");
  }
  // On sf, per segment s: fetch(s) into window s&1, summaries of its
  // blocks, then the selection and plan of s+1 (they need those summaries);
  // only then is the attention of s released on sa, so that the small
  // selection kernels do not share the CUs with it.  fetch(s+1) then runs
  // beside attention(s); it waits for attention(s-1), the last reader of its
  // window.
  const int nseg = p.S / p.L;
  if ((rc = tier_plan_step(p, 0, q, summ, sel, t, 0, sf))) return rc;
  for (int seg = 0; seg < nseg; ++seg) {
    const int w = seg & 1;
    if (two && seg >= 2 && (e = hipStreamWaitEvent(sf, ev[2 + w], 0)) != hipSuccess)
      return hip_fail(e, "stream wait");
    e = hga::launch_tier_fetch(p, kh, vh, t.list[w], t.count[w], seg, t.kw[w], t.vw[w], sf);
    if (e != hipSuccess) return hip_fail(e, "tier fetch launch");
    if ((rc = tier_summarize(p, seg, summ, t, w, sf))) return rc;
    if (seg + 1 < nseg && (rc = tier_plan_step(p, seg + 1, q, summ, sel, t, w ^ 1, sf)))
      return rc;
    if (two) {
      if ((e = hipEventRecord(ev[w], sf)) != hipSuccess) return hip_fail(e, "event record");
      if ((e = hipStreamWaitEvent(sa, ev[w], 0)) != hipSuccess) return hip_fail(e, "stream wait");
    }
    if ((rc = tier_attn_step(p, seg, bwd, q, dO, o, lse, dq, dk, dv, t, w, sa))) return rc;
    if (two && (e = hipEventRecord(ev[2 + w], sa)) != hipSuccess)
      return hip_fail(e, "event record");
  }
  // stream waited for every fetch-stream launch (the last fetch's event)
  return ok();
}

int hga_segment_pass(const hga_config* cfg, int32_t flags, const void* q, const void* k,
                     const void* v, const void* dO, float* summ, int32_t* sel, void* o,
                     float* lse, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     void* stream, void* stream2) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if (flags & HGA_STEP_SUMMARIES_READY)
    return fail(HGA_ERR_ARG, "the pass summarizes the history itself");
  if ((rc = check_step_args(p, flags, q, k, v, dO, summ, sel, o, lse, dq, dk, dv, ws, ws_bytes,
                            pass_workspace_bytes(p))))
    return rc;
  const bool bwd = (flags & HGA_STEP_BWD) != 0;
  const bool two = stream2 != nullptr;
  hipStream_t st[2] = {(hipStream_t)stream, two ? (hipStream_t)stream2 : (hipStream_t)stream};
  const int nseg = p.S / p.L;
  hipError_t e;
  // every block a later segment can select, once
  if (nseg > 1) {
    e = hga::launch_summarize(p, k, 0, (p.S - p.L) / p.Bh, summ, st[0]);
    if (e != hipSuccess) return hip_fail(e, "summarize launch");
  }
  if (p.dtype == HGA_BF16) {
    // one selection launch, one forward launch (it also writes each
    // segment's delta rows), one dK/dV launch and one dQ launch, each over
    // all segments: no per-segment launch tails, and the second stream is
    // not needed
    const size_t dstride = hga::bwd_delta_bytes(p);
    float* delta = (float*)ws;
    e = hga::launch_select_pass(p, q, summ, 0, nseg, sel, st[0]);
    if (e != hipSuccess) return hip_fail(e, "select launch");
    e = hga::launch_fwd_pass(p, q, k, v, sel, 0, nseg, o, lse, st[0], bwd ? dO : nullptr,
                             bwd ? delta : nullptr, dstride);
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    if (bwd) {
      e = hga::launch_bwd_pass(p, q, k, v, lse, dO, sel, 0, nseg, dq, dk, dv, delta, dstride,
                               st[0]);
      if (e != hipSuccess) return hip_fail(e, "backward launch");
    }
    return ok();
  }
  // f32: whole steps, alternating between the two streams
  const size_t one = round256(hga::bwd_workspace_bytes(p));
  void* wsp[2] = {ws, two && ws ? (void*)((char*)ws + one) : ws};
  hipEvent_t ev_in = nullptr, ev_out = nullptr;
  if (two) {
    if ((e = pass_events(&ev_in, &ev_out)) != hipSuccess) return hip_fail(e, "event create");
    if ((e = hipEventRecord(ev_in, st[0])) != hipSuccess) return hip_fail(e, "event record");
    if ((e = hipStreamWaitEvent(st[1], ev_in, 0)) != hipSuccess) return hip_fail(e, "stream wait");
  }
  for (int seg = 0; seg < nseg; ++seg) {
    const int i = seg & 1;
    if ((rc = run_step(p, seg, flags | HGA_STEP_SUMMARIES_READY, q, k, v, dO, summ, sel, o, lse,
                       dq, dk, dv, wsp[i], st[i])))
      return rc;
  }
  if (two) {
    if ((e = hipEventRecord(ev_out, st[1])) != hipSuccess) return hip_fail(e, "event record");
    if ((e = hipStreamWaitEvent(st[0], ev_out, 0)) != hipSuccess) return hip_fail(e, "stream wait");
  }
  return ok();
}

int hga_segment_pass_noalloc(const hga_config* cfg, int32_t flags, const void* q, const void* k,
                             const void* v, const void* dO, float* summ, int32_t* sel, void* o,
                             float* lse, void* dq, void* dk, void* dv, void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  // hga_segment_pass's argument checks (the workspace aside), before the
  // scratch array is looked up
  if (flags & ~HGA_STEP_BWD)
    return fail(HGA_ERR_ARG, "unknown flags 0x%x (the pass summarizes the history itself)",
                flags);
  HGA_REQUIRE(q);
  HGA_REQUIRE(k);
  HGA_REQUIRE(v);
  HGA_REQUIRE(summ);
  HGA_REQUIRE(sel);
  HGA_REQUIRE(o);
  if (flags & HGA_STEP_BWD) {
    HGA_REQUIRE(lse);
    HGA_REQUIRE(dO);
    HGA_REQUIRE(dq);
    HGA_REQUIRE(dk);
    HGA_REQUIRE(dv);
  }
  // the scratch hga_segment_pass would take from its workspace argument
  const size_t need = (flags & HGA_STEP_BWD) ? pass_workspace_bytes(p) : 0;
  if (need > kNoallocScratchBytes)
    return fail(HGA_ERR_WORKSPACE,
                "the pass needs %zu bytes of scratch; the no-allocation form holds %zu per GPU",
                need, kNoallocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
  }
  return hga_segment_pass(cfg, flags, q, k, v, dO, summ, sel, o, lse, dq, dk, dv, ws, need,
                          stream, nullptr);
}

int hga_segment_step_exact(const hga_config* cfg, int32_t seg, const void* q, const void* k,
                           const void* v, const void* dO, const float* summ, int32_t* sel,
                           void* o, float* lse, void* dq, void* dk, void* dv, float* hist_dk,
                           float* hist_dv, void* ws, size_t ws_bytes, void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if ((rc = check_seg(p, seg))) return rc;
  if (p.dtype != HGA_BF16)
    return fail(HGA_ERR_UNSUPPORTED, "the exact-gradient step needs bf16");
  if (p.nqb > 64 || p.nqb * p.K > hga::kHistMaxEntries)
    return fail(HGA_ERR_UNSUPPORTED,
                "the exact-gradient step needs seg_len/query_block <= 64 and "
                "(seg_len/query_block)*top_k <= %d", hga::kHistMaxEntries);
  HGA_REQUIRE(q);
  HGA_REQUIRE(k);
  HGA_REQUIRE(v);
  HGA_REQUIRE(dO);
  HGA_REQUIRE(summ);
  HGA_REQUIRE(sel);
  HGA_REQUIRE(o);
  HGA_REQUIRE(lse);
  HGA_REQUIRE(dq);
  HGA_REQUIRE(dk);
  HGA_REQUIRE(dv);
  HGA_REQUIRE(hist_dk);
  HGA_REQUIRE(hist_dv);
  HGA_REQUIRE(ws);
  const size_t need = hga::bwd_exact_workspace_bytes(p);
  if (ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hga::launch_select(p, q, summ, seg, sel, st);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  const bool fuse = hga::fused_delta(p);
  e = hga::launch_fwd(p, q, k, v, sel, seg, o, lse, st, fuse ? dO : nullptr,
                      fuse ? (float*)ws : nullptr);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  e = hga::launch_bwd(p, q, k, v, o, lse, dO, sel, seg, dq, dk, dv, (float*)ws, st, fuse,
                      hist_dk, hist_dv);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

int hga_segment_pass_exact(const hga_config* cfg, const void* q, const void* k, const void* v,
                           const void* dO, float* summ, int32_t* sel, void* o, float* lse,
                           void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                           void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if (p.dtype != HGA_BF16)
    return fail(HGA_ERR_UNSUPPORTED, "the exact-gradient pass needs bf16");
  if (p.nqb > 64 || p.nqb * p.K > hga::kHistMaxEntries)
    return fail(HGA_ERR_UNSUPPORTED,
                "the exact-gradient pass needs seg_len/query_block <= 64 and "
                "(seg_len/query_block)*top_k <= %d", hga::kHistMaxEntries);
  HGA_REQUIRE(q);
  HGA_REQUIRE(k);
  HGA_REQUIRE(v);
  HGA_REQUIRE(dO);
  HGA_REQUIRE(summ);
  HGA_REQUIRE(sel);
  HGA_REQUIRE(o);
  HGA_REQUIRE(lse);
  HGA_REQUIRE(dq);
  HGA_REQUIRE(dk);
  HGA_REQUIRE(dv);
  HGA_REQUIRE(ws);
  const size_t need = pass_exact_workspace_bytes(p);
  if (ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  const int nseg = p.S / p.L;
  const size_t dstride = hga::bwd_delta_bytes(p);
  const size_t nsum = (size_t)p.B * p.Hkv * p.S * p.D;
  float* delta = (float*)ws;
  float* hist_dk = (float*)((char*)ws + (size_t)nseg * dstride);
  float* hist_dv = (float*)((char*)hist_dk + round256(nsum * sizeof(float)));
  void* list_ws = (char*)hist_dv + round256(nsum * sizeof(float));
  hipError_t e;
  if (nseg > 1) {
    e = hga::launch_summarize(p, k, 0, (p.S - p.L) / p.Bh, summ, st);
    if (e != hipSuccess) return hip_fail(e, "summarize launch");
  }
  e = hga::launch_select_pass(p, q, summ, 0, nseg, sel, st);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  e = hga::launch_fwd_pass(p, q, k, v, sel, 0, nseg, o, lse, st, dO, delta, dstride);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  // history sums: each segment's queries add their part to the rows of the
  // blocks they selected, from the last segment to the first (a fixed order)
  if ((e = hga::launch_zero(hist_dk, nsum, st)) != hipSuccess) return hip_fail(e, "zero launch");
  if ((e = hga::launch_zero(hist_dv, nsum, st)) != hipSuccess) return hip_fail(e, "zero launch");
  // every segment's list of selected blocks in one launch
  if ((e = hga::launch_hist_lists(p, sel, list_ws, st)) != hipSuccess)
    return hip_fail(e, "history list launch");
  for (int seg = nseg - 1; seg >= 1; --seg) {
    e = hga::launch_hist_exact(p, q, k, v, lse, dO, sel, seg,
                               (const float*)((const char*)delta + (size_t)seg * dstride),
                               hist_dk, hist_dv, list_ws, st);
    if (e != hipSuccess) return hip_fail(e, "history backward launch");
  }
  // local dK/dV of every segment plus its rows' history sums, and dQ
  e = hga::launch_bwd_pass(p, q, k, v, lse, dO, sel, 0, nseg, dq, dk, dv, delta, dstride, st,
                           hist_dk, hist_dv);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

int hga_decode_step(const hga_config* cfg, int32_t pos, int32_t n, const void* q,
                    const void* k, const void* v, float* summ, int32_t* sel, void* o,
                    float* lse, void* ws, size_t ws_bytes, void* stream) {
  hga::Prob p;
  int rc = make_prob(cfg, &p);
  if (rc) return rc;
  if (n < 1 || pos < 0 || (int64_t)pos + n > p.S)
    return fail(HGA_ERR_ARG, "tokens [%d, %d + %d) outside [0, %d)", pos, pos, n, p.S);
  if (pos / p.L != (pos + n - 1) / p.L)
    return fail(HGA_ERR_ARG, "tokens [%d, %d) cross a segment boundary (seg_len %d)", pos,
                pos + n, p.L);
  if (p.G * n > hga::decode_max_rows())
    return fail(HGA_ERR_UNSUPPORTED, "G*n = %d exceeds %d query rows per KV head", p.G * n,
                hga::decode_max_rows());
  HGA_REQUIRE(q);
  HGA_REQUIRE(k);
  HGA_REQUIRE(v);
  HGA_REQUIRE(summ);
  HGA_REQUIRE(sel);
  HGA_REQUIRE(o);
  HGA_REQUIRE(ws);
  const size_t need = hga::decode_workspace_bytes(p);
  if (ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  const int t0 = pos / p.L * p.L;
  hipError_t e;
  if (pos == t0 && t0 > 0) {
    // the first tokens of a segment: the previous segment's blocks become history
    e = hga::launch_summarize(p, k, (t0 - p.L) / p.Bh, t0 / p.Bh, summ, st);
    if (e != hipSuccess) return hip_fail(e, "summarize launch");
  }
  // bf16 with k < history blocks <= 1024: scores (each scoring block also
  // keeps its own k best), attention (whose history chunks finish the top-k
  // from those lists), merge; else selection, attention, merge
  const bool fused = hga::decode_fused(p, pos, n);
  e = hga::launch_select_decode(p, q, n, t0, summ, sel, hga::decode_score_ws(p, ws), st,
                                fused ? hga::decode_cand_score_ws(p, ws) : nullptr,
                                fused ? hga::decode_cand_idx_ws(p, ws) : nullptr);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  e = hga::launch_decode(p, pos, n, q, k, v, sel, o, lse, (float*)ws, fused, st);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

int hga_profile_begin(uint32_t mask) {
  g_prof_on = true;
  g_prof_mask = mask;
  return ok();
}

int hga_profile_end(double* ms, int64_t* count) {
  if (ms == nullptr || count == nullptr) return fail(HGA_ERR_ARG, "ms/count is NULL");
  for (int i = 0; i < HGA_KCLASS_COUNT; ++i) { ms[i] = 0.0; count[i] = 0; }
  int rc = HGA_OK;
  for (const ProfEvent& ev : g_prof_events) {
    if (rc == HGA_OK) {
      hipError_t e = hipEventSynchronize(ev.stop);
      float t = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&t, ev.start, ev.stop);
      if (e != hipSuccess) {
        rc = hip_fail(e, "profiling event");
      } else if (ev.kclass >= 0 && ev.kclass < HGA_KCLASS_COUNT) {
        ms[ev.kclass] += t;
        count[ev.kclass] += 1;
      }
    }
    g_prof_pool.push_back(ev.start);
    g_prof_pool.push_back(ev.stop);
  }
  g_prof_events.clear();
  g_prof_on = false;
  for (hipEvent_t e : g_prof_pool) hipEventDestroy(e);
  g_prof_pool.clear();
  if (rc == HGA_OK) ok();
  return rc;
}

}  // extern "C"
