/*
 * hga.h - C ABI of the Hierarchical Global Attention (HGA) hot path with
 * segmented backpropagation, for AMD Instinct MI355X (gfx950).
 *
 * Page keys used in citations:
 *   [JA] 「低VRAM長文脈ファインチューニング：階層的グローバル注意と分割バック
 *        プロpagationの実践」, sns.style (Japanese edition)
 *   [FR] « Ajustement fin long-contexte à faible VRAM : une approche
 *        d'optimisation avec attention globale hiérarchique », sns.style
 *   [DE] „Geringer-VRAM Lang-Kontext Fine-Tuning: Hierarchische globale
 *        Aufmerksamkeit und segmentierte Rückwärtsausbreitung in der
 *        Praxis", sns.style (German edition)
 *   [KO] 「저VRAM 긴 컨텍스트 미세조정: 계층적 글로벌 주의와 분할 역전파의
 *        실전 적용」, sns.style (Korean edition)
 *   [SeCO] notes on "Training Long-Context LLMs Efficiently via Chunk-wise
 *        Optimization", f-binder
 *
 * The method ([JA] 背景と概要; [FR] Contexte, Analyse approfondie): a long
 * sequence is processed segment by segment; only the active segment is
 * differentiable and history KV is detached; resident per-block summaries
 * of the history stay on the GPU ([JA] 深掘り分析); for every query block
 * a bounded, exact set of history tokens is loaded and attended together
 * with the active segment.  The summary is the mean key of a block per KV
 * head, the score is its dot product with the query block's mean query, and
 * top-k ties go to the lower block index.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Shapes: B batch, S sequence length, L segment length, Bh history block,
 *  Bq query block, k top-k, Hq query heads, Hkv KV heads, G = Hq/Hkv,
 *  D head dim.  Query head h reads KV head h / G.
 *  Segment s covers tokens [s*L, (s+1)*L); its history is the whole blocks
 *  [0, s*L/Bh); it has L/Bq query blocks.
 *
 *  Layouts (all row-major, dense, device memory, allocated by the caller):
 *    q, o, dO, dq      [B, Hq,  S, D]        dtype of the config
 *    k, v, dk, dv      [B, Hkv, S, D]        dtype of the config
 *    lse               [B, Hq,  S]           float32, natural log
 *    summ              [B, Hkv, S/Bh, D]     float32 block-mean keys
 *    sel               [B, Hkv, S/Bq, k]     int32, ascending, -1 padded
 *  Every call reads and writes only the rows of the segment it is given
 *  (history K/V and summaries are read as well).  Gradients are written,
 *  not accumulated.  Work is enqueued on `stream` (a hipStream_t, NULL =
 *  the default stream); no entry point synchronizes or allocates device
 *  memory.  State kept between calls: the optional profiling hooks at the
 *  end of this file, and the timing-free HIP events that hga_segment_pass
 *  (f32) and hga_segment_pass_host use to hand work between their two
 *  streams -- created on a calling thread's first such call on a device,
 *  kept for that thread and device and reused by its later calls, never
 *  freed; and the scratch array of hga_segment_pass_noalloc, one per GPU,
 *  which holds the last call's intermediate values.  Every other entry
 *  point keeps nothing.  Scratch space comes from
 *  `ws`, of at least hga_workspace_size() bytes.  Results are bitwise deterministic
 *  (no floating-point atomics).
 *
 *  Errors: every entry point returns HGA_OK (0) or a negative code.  The
 *  arguments are validated on the host before anything is enqueued; on an
 *  error nothing is enqueued and hga_last_error() returns a message
 *  (thread-local, valid until the next call on the same thread).  No C++
 *  exception crosses this interface.
 */
#ifndef HGA_H
#define HGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HGA_OK = 0,
  HGA_ERR_ARG = -1,          /* null pointer, bad size or index           */
  HGA_ERR_UNSUPPORTED = -2,  /* dtype, head_dim or size the kernels lack  */
  HGA_ERR_WORKSPACE = -3,    /* ws too small                               */
  HGA_ERR_HIP = -4           /* a HIP runtime call or launch failed        */
};

typedef enum { HGA_F32 = 0, HGA_BF16 = 1 } hga_dtype;

/* One attention layer's HGA problem.  Requirements (else HGA_ERR_ARG):
 * all sizes >= 1, S % L == 0, L % Bh == 0, L % Bq == 0, Hq % Hkv == 0.
 * Supported (else HGA_ERR_UNSUPPORTED): head_dim 64 or 128; dtype F32 or
 * BF16; S/Bh <= 8192; top_k <= 1024; bf16 kernels need Bh and Bq to be
 * multiples of 16; one head's S x D slice at most 2 GiB. */
typedef struct hga_config {
  int32_t batch;
  int32_t seq_len;
  int32_t seg_len;
  int32_t hist_block;
  int32_t query_block;
  int32_t top_k;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;          /* hga_dtype */
  float softmax_scale;    /* <= 0 selects 1/sqrt(head_dim) */
} hga_config;

/* a1 - resident block summaries ([JA] 深掘り分析: per-block summaries of the
 * history stay resident and grow with length).
 * summ[b,g,i,:] = (1/Bh) * sum over the Bh keys of block i of k[b,g,t,:],
 * for blk_begin <= i < blk_end (0 <= blk_begin <= blk_end <= S/Bh).
 * Accumulates in float32.  Other rows of summ are left untouched. */
int hga_summarize(const hga_config* cfg, const void* k, int32_t blk_begin,
                  int32_t blk_end, float* summ, void* stream);

/* a2 + a3 - query-block mean and top-k selection for segment `seg`
 * ([JA] 背景と概要: a bounded set of history tokens per query block;
 * [FR] Contexte: targeted loading of a bounded set of relevant tokens).
 * For every (b, g, query block j): qbar = mean of q over the G query heads
 * of group g and the Bq tokens of the block (float32); score_i = qbar .
 * summ[b,g,i,:] for the nb = seg*L/Bh history blocks; if nb <= k all blocks
 * are taken, else the k best by (score descending, index ascending).  The
 * chosen indices are written ascending to sel[b,g,seg*L/Bq + j, :] and
 * padded with -1.  Reads summ rows [0, nb), which must be current. */
int hga_select(const hga_config* cfg, const void* q, const float* summ,
               int32_t seg, int32_t* sel, void* stream);

/* a4 - standalone block-sparse gather of the selected history K and V of
 * segment `seg` ([FR] Analyse approfondie: targeted loading of the chosen
 * history tokens rather than a full scan).  k_out and v_out are
 * [B, Hkv, L/Bq, k, Bh, D] in the config dtype; slot t of query block j
 * receives block sel[b,g,seg*L/Bq+j,t] of k (resp. v), or zeros when that
 * entry is -1.  The attention kernels below read the same blocks directly
 * and do not need this copy; it exists to measure and check the gather. */
int hga_gather(const hga_config* cfg, const void* k, const void* v,
               const int32_t* sel, int32_t seg, void* k_out, void* v_out,
               void* stream);

/* a5 - forward attention of segment `seg` ([JA] 背景と概要: exact attention
 * over the bounded history set; [DE]/[KO] same).  For each (b, h, t) of
 * the segment, the key set is the tokens of the selected blocks of
 * (b, h/G, query block of t) together with the local tokens seg*L .. t;
 * one softmax with scale over that joint set; o = softmax . v, lse = log of
 * the softmax denominator (natural log, including the scale).  `lse` may
 * be NULL (inference).  ws: hga_workspace_size(cfg, HGA_OP_FWD) bytes
 * (currently 0; ws may be NULL). */
int hga_attn_fwd(const hga_config* cfg, const void* q, const void* k,
                 const void* v, const int32_t* sel, int32_t seg, void* o,
                 float* lse, void* ws, size_t ws_bytes, void* stream);

/* a6 + a7 + a8 - backward of segment `seg` for the loss whose gradient
 * with respect to o is dO ([FR] Analyse approfondie: only the active
 * segment's gradients are computed; history KV is detached).
 *   delta = rowsum(dO * o);  p = exp(scale*q.k - lse);
 *   dS = p * (dO.v - delta);  dq = scale * sum dS k   (history and local);
 *   dk[t'] = scale * sum dS q, dv[t'] = sum p dO, for local keys t' only,
 *   summed over the queries t >= t' of the segment and the G heads.
 * History rows of dk/dv are not written.  ws: hga_workspace_size(cfg,
 * HGA_OP_BWD) bytes, caller-owned scratch that the call overwrites: delta
 * [B, Hq, L] fp32, then fp32 partial sums of dk/dv for key tiles whose work
 * is split between two blocks (added in a fixed order, so results stay
 * bitwise deterministic).  Calls that share one workspace must not overlap. */
int hga_attn_bwd(const hga_config* cfg, const void* q, const void* k,
                 const void* v, const void* o, const float* lse,
                 const void* dO, const int32_t* sel, int32_t seg, void* dq,
                 void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);

/* a9 - one step of the segment loop ([FR] Analyse approfondie: segments
 * processed one after another): summarize the blocks that segment seg-1
 * closed (none for seg 0), select, forward, and with HGA_STEP_BWD the
 * backward.  Calling it for seg = 0, 1, ..., S/L-1 in order runs the whole
 * segmented pass; summ must hold the blocks of earlier segments (which the
 * earlier steps wrote).  dO, dq, dk, dv may be NULL without HGA_STEP_BWD;
 * lse may be NULL without HGA_STEP_BWD.  ws: hga_workspace_size(cfg,
 * HGA_OP_STEP) bytes. */
/* HGA_STEP_SUMMARIES_READY: summ already holds every block before the
 * segment; the step skips its summarize. */
enum { HGA_STEP_BWD = 1, HGA_STEP_SUMMARIES_READY = 2 };
int hga_segment_step(const hga_config* cfg, int32_t seg, int32_t flags,
                     const void* q, const void* k, const void* v,
                     const void* dO, float* summ, int32_t* sel, void* o,
                     float* lse, void* dq, void* dk, void* dv, void* ws,
                     size_t ws_bytes, void* stream);

/* Decode step for n new tokens at positions pos .. pos+n-1, all inside one
 * segment (t0 = floor(pos/L)*L) ([JA] 深掘り分析: inference over up to
 * 131,072 tokens with the resident summaries growing; [JA] 業界への影響 and
 * [FR] Contexte: HGA as a module for retrieval and generation).  The pages
 * give no decode procedure; the new tokens are read as one query block of
 * their segment:
 *   - if pos == t0 > 0, the L/Bh blocks of the previous segment are
 *     summarized into summ first (as hga_segment_step does); summ rows
 *     [0, t0/Bh) must otherwise be current;
 *   - qbar = mean of q over the G heads of a group and the n tokens; the k
 *     best history blocks before t0 by (score desc, index asc), or all of
 *     them, are written ascending, -1 padded, to sel[b,g,:];
 *   - token pos+i attends, with one softmax, to the selected history
 *     tokens and the local tokens t0 .. pos+i.
 * Layouts: q and o [B, Hq, n, D] (dtype of the config, dense), lse
 * [B, Hq, n] float32 natural log (may be NULL), sel [B, Hkv, k] int32; k and
 * v are the full [B, Hkv, S, D] caches holding every token up to pos+n-1.
 * Requirements: 0 <= pos, n >= 1, pos+n <= S, the n tokens in one segment
 * (else HGA_ERR_ARG); G*n <= 64 (else HGA_ERR_UNSUPPORTED).  ws:
 * hga_workspace_size(cfg, HGA_OP_DECODE) bytes of scratch (per-chunk
 * partial sums, combined in a fixed order: results are deterministic; the
 * selection scores and top-k candidate lists); calls sharing a workspace
 * must not overlap.  bf16 steps with k < t0/Bh <= 1024 and k <= 256 run as
 * three launches: the scores, where every block of 128 candidates (256
 * when 128-candidate lists would leave over 1,024 entries) also keeps its
 * own k best; the attention, whose history chunks pick the k best
 * of those lists (the k best of the union, by the same rule); the merge.
 * The others run as three or four launches (selection, attention, merge). */
int hga_decode_step(const hga_config* cfg, int32_t pos, int32_t n, const void* q,
                    const void* k, const void* v, float* summ, int32_t* sel, void* o,
                    float* lse, void* ws, size_t ws_bytes, void* stream);

/* Exact-gradient form of hga_segment_step with the backward ([SeCO] 提案手法:
 * the forward keeps each chunk's KV; the backward visits the chunks from
 * the last one, rebuilding one chunk's graph at a time, and the gradient is
 * exact).  History is not detached: the keys and values of the blocks a
 * segment's query blocks selected also receive those queries' gradient
 * (the selection itself, being discrete, receives none).
 *   - summ must hold every block before the segment (call hga_summarize
 *     over [0, S/Bh) first; this step summarizes nothing);
 *   - hist_dk, hist_dv: float32 [B, Hkv, S, D], zeroed by the caller before
 *     the first step; the steps must visit the segments in descending
 *     order.  Step seg adds scale * sum dS q (dk) and sum P dO (dv) of its
 *     queries into the rows of the history blocks they selected, and writes
 *     dk/dv of its own rows as its local part plus the sums later segments
 *     left in those rows (complete, since later segments came first);
 *   - select, forward and dq are those of hga_segment_step.
 * Requirements: bf16 (else HGA_ERR_UNSUPPORTED); L/Bq <= 64 and
 * (L/Bq)*k <= 8192 (else HGA_ERR_UNSUPPORTED).  ws:
 * hga_workspace_size(cfg, HGA_OP_STEP_EXACT) bytes.  Results are
 * deterministic (every row has one writer per step; no atomics). */
int hga_segment_step_exact(const hga_config* cfg, int32_t seg, const void* q, const void* k,
                           const void* v, const void* dO, const float* summ, int32_t* sel,
                           void* o, float* lse, void* dq, void* dk, void* dv, float* hist_dk,
                           float* hist_dv, void* ws, size_t ws_bytes, void* stream);

/* The whole segmented pass: hga_summarize over every block a later segment
 * can select (once, on `stream`), then select, forward and (flags
 * HGA_STEP_BWD) backward of seg = 0 .. S/L-1.  Once the summaries exist the
 * segments are independent: each reads only the inputs and those summaries
 * and writes rows of its own.
 *   - bf16: one selection launch, one forward launch (which also writes
 *     every segment's delta rows), one dK/dV launch and one dQ launch, each
 *     over all segments, so no launch has a per-segment tail.  The forward
 *     and dQ blocks walk all keys of their query rows themselves, so float
 *     sums are added in another order than in hga_segment_step: equal within
 *     rounding, not bit for bit (selections are identical).  stream2 is not
 *     used.
 *   - f32: hga_segment_step per segment (without its summarize); with
 *     stream2 non-NULL the segments alternate between stream and stream2
 *     (stream2 first waits for the summaries), which fills the CUs one
 *     segment's kernels leave idle near their ends; results equal the
 *     one-stream pass's bit for bit.
 * When the call returns, everything it enqueued is ordered before later work
 * on `stream`.  Both streams must be at default priority.  flags:
 * HGA_STEP_BWD or 0.  ws: hga_workspace_size(cfg, HGA_OP_PASS) bytes
 * (needed with HGA_STEP_BWD; bf16: every segment's delta rows).  The library keeps two
 * timing-free HIP events per calling thread and device for the f32 hand-offs. */
int hga_segment_pass(const hga_config* cfg, int32_t flags, const void* q, const void* k,
                     const void* v, const void* dO, float* summ, int32_t* sel, void* o,
                     float* lse, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     void* stream, void* stream2);

/* hga_segment_pass without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The scratch space hga_segment_pass takes
 * from `ws` (hga_workspace_size(cfg, HGA_OP_PASS) bytes, needed with
 * HGA_STEP_BWD) comes instead from a fixed array of
 * HGA_NOALLOC_SCRATCH_BYTES (64 MiB) in device memory that the library holds
 * on every GPU it runs on, from the code object's load until the process
 * ends; at train_16k the pass needs 2 MiB of it, at 4 x 32K 16 MiB.  Larger
 * needs return HGA_ERR_WORKSPACE before anything is enqueued.  Everything
 * runs on `stream` (the f32 pass does not use a second stream here, so no
 * event is created either); the call makes no hipMalloc, hipFree or other
 * allocating call.  The array keeps the last call's contents and nothing in
 * it needs to start at zero.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must not be made; calls ordered on one stream are fine.  Results
 * equal hga_segment_pass's (same kernels, same order) bit for bit.  Other
 * arguments, requirements and errors as hga_segment_pass. */
#define HGA_NOALLOC_SCRATCH_BYTES (64u << 20)
int hga_segment_pass_noalloc(const hga_config* cfg, int32_t flags, const void* q, const void* k,
                             const void* v, const void* dO, float* summ, int32_t* sel, void* o,
                             float* lse, void* dq, void* dk, void* dv, void* stream);

/* The whole exact-gradient pass ([SeCO] 提案手法: the backward visits the
 * chunks from the last one and the gradient is exact; here the history
 * keys are not detached): hga_summarize over every block a later segment
 * can select, the selection and forward of every segment (one launch
 * each), then the backward: each segment's queries, from the last segment
 * to the first, add their dK/dV for the history blocks they selected into
 * fp32 sums kept in ws; then one dK/dV launch writes every segment's local
 * part plus its rows' sums, and one launch writes dQ.  The same results as
 * hga_segment_step_exact called for seg = S/L-1 .. 0 after hga_summarize,
 * within rounding (float sums in another order).  dq, dk, dv: the complete
 * gradient of the layer's attention with respect to q, k, v.
 * Requirements: bf16 (else HGA_ERR_UNSUPPORTED); L/Bq <= 64 and
 * (L/Bq)*k <= 8192 (else HGA_ERR_UNSUPPORTED).  ws:
 * hga_workspace_size(cfg, HGA_OP_PASS_EXACT) bytes (every segment's delta
 * rows, the fp32 history sums of dK and dV, every segment's history block
 * list).
 * Results are deterministic (every sum has one writer at a time; no
 * atomics on floats). */
int hga_segment_pass_exact(const hga_config* cfg, const void* q, const void* k, const void* v,
                           const void* dO, float* summ, int32_t* sel, void* o, float* lse,
                           void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                           void* stream);

/* Host-RAM history tier ([JA] 背景と概要 and [FR] Contexte: the history KV
 * is moved off the GPU to system RAM, and only the active segment's state
 * stays in GPU memory; [JA] 深掘り分析: the block summaries stay resident,
 * so the limit becomes host capacity; [JA] 今後の展望 and [FR]
 * Perspectives: the transfers between GPU and host memory are the part to
 * optimise).  hga_segment_step with the keys and values in host memory:
 *   - k_host, v_host: [B, Hkv, S, D] bf16 in pinned host memory (hipHostMalloc,
 *     or a pinned torch tensor), read by the GPU directly; rows 0 .. t0+L-1
 *     must hold the keys / values (t0 = seg*L).  Never written.
 *   - per step, on the GPU: the selection is made as in hga_segment_step
 *     (summ must hold the blocks before t0), then the union of the blocks the
 *     segment's query blocks chose (per (b, g), at most
 *     C = min((L/Bq)*k, (S-L)/Bh) blocks) and the segment's own L rows are
 *     copied from host memory into a window in ws of C*Bh + L rows per
 *     (b, g); forward and backward read the window, and the summaries of
 *     the segment's own blocks (history of the later segments; none for the
 *     last segment) are taken from the window into summ, unless
 *     HGA_STEP_SUMMARIES_READY.  The host never waits for the selection.
 *   - every other argument, and every result, is that of hga_segment_step:
 *     o, lse, dq, dk, dv and sel equal its results bit for bit (the window
 *     keeps the chosen blocks in ascending order), and after the steps of
 *     segments 0 .. S/L-1 in order so does summ.
 * HBM use per step is bounded by the window, whatever S is; the tier needs
 * host memory for K and V only.  Requirements: bf16 (else
 * HGA_ERR_UNSUPPORTED); k_host and v_host pinned host memory (else
 * HGA_ERR_ARG).  ws: hga_workspace_size(cfg, HGA_OP_STEP_HOST) bytes (also
 * without HGA_STEP_BWD); calls sharing a workspace must not overlap. */
int hga_segment_step_host(const hga_config* cfg, int32_t seg, int32_t flags, const void* q,
                          const void* k_host, const void* v_host, const void* dO, float* summ,
                          int32_t* sel, void* o, float* lse, void* dq, void* dk, void* dv,
                          void* ws, size_t ws_bytes, void* stream);

/* The whole segmented pass with the host tier: hga_segment_step_host for
 * seg = 0 .. S/L-1, with two windows in ws.  The selections, summaries and
 * fetches run on stream2, the attention on stream: the fetch of segment
 * seg+1 runs while the attention of segment seg does (the selection of
 * seg+1 comes before that attention starts), and waits only for the
 * attention of seg-1, the last reader of its window (stream2 NULL:
 * everything on stream, in order).  The overlap needs the two streams on
 * different hardware queues: HIP runs streams on a few of them
 * (GPU_MAX_HW_QUEUES, four by default), and streams that share one run one
 * after the other (results are the same, only slower).  Results equal the
 * steps' bit for bit.  When the call returns,
 * everything it enqueued is ordered before later work on `stream`; both
 * streams at default priority.  flags: HGA_STEP_BWD or 0.  ws:
 * hga_workspace_size(cfg, HGA_OP_PASS_HOST) bytes.  The library keeps five
 * timing-free HIP events per calling thread and device for the hand-offs. */
int hga_segment_pass_host(const hga_config* cfg, int32_t flags, const void* q,
                          const void* k_host, const void* v_host, const void* dO, float* summ,
                          int32_t* sel, void* o, float* lse, void* dq, void* dk, void* dv,
                          void* ws, size_t ws_bytes, void* stream, void* stream2);

/* Workspace bytes for an operation (0 if none is needed), or 0 with
 * hga_last_error() set if the config is invalid. */
enum { HGA_OP_FWD = 0, HGA_OP_BWD = 1, HGA_OP_STEP = 2, HGA_OP_DECODE = 3,
       HGA_OP_STEP_EXACT = 4, HGA_OP_PASS = 5, HGA_OP_PASS_EXACT = 6,
       HGA_OP_STEP_HOST = 7, HGA_OP_PASS_HOST = 8 };
size_t hga_workspace_size(const hga_config* cfg, int32_t op);

/* Message of the last failure on this thread ("" if none). */
const char* hga_last_error(void);

/* Library version string. */
const char* hga_version(void);

/* ---- optional profiling hooks (timing only, never change results) ----
 * hga_profile_begin(mask) makes later launches on this thread of each kernel
 * whose class bit (1 << class) is set in mask carry a HIP start / stop event
 * pair that the kernel's own dispatch stamps (hipExtLaunchKernel), so the
 * timing adds nothing between kernels on the stream.  hga_profile_end() waits for those events,
 * writes per-class total milliseconds and launch counts into ms[] and
 * count[] (arrays of HGA_KCLASS_COUNT entries), stops recording and
 * releases the events.  Kernel classes: */
enum {
  HGA_K_SUMMARIZE = 0,
  HGA_K_SELECT = 1,
  HGA_K_GATHER = 2,
  HGA_K_FWD = 3,
  HGA_K_BWD_PRE = 4,
  HGA_K_BWD_DQ = 5,
  HGA_K_BWD_DKDV = 6,
  HGA_K_DECODE = 7,
  HGA_K_DECODE_MERGE = 8,
  HGA_K_BWD_HIST = 9,
  HGA_K_TIER_PLAN = 10,
  HGA_K_TIER_FETCH = 11,
  HGA_KCLASS_COUNT = 12
};
int hga_profile_begin(uint32_t mask);
int hga_profile_end(double* ms, int64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H */
