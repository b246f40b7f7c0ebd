"""HGA oracle, vectorized form: plain, slow, fp64 CPU implementation.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP library and never imports it.

Page keys used in citations:
  [JA] 「低VRAM長文脈ファインチューニング：階層的グローバル注意と分割バック
       プロpagationの実践」, sns.style (Japanese edition); sections
       背景と概要 (background), 深掘り分析 (analysis)
  [DE] „Geringer-VRAM Lang-Kontext Fine-Tuning: Hierarchische globale
       Aufmerksamkeit und segmentierte Rückwärtsausbreitung in der Praxis",
       sns.style (German edition); sections Hintergrund, Tiefenanalyse
  [FR] « Ajustement fin long-contexte à faible VRAM : une approche
       d'optimisation avec attention globale hiérarchique », sns.style;
       sections Contexte, Analyse approfondie
  [KO] 「저VRAM 긴 컨텍스트 미세조정: 계층적 글로벌 주의와 분할 역전파의
       실전 적용」, sns.style (Korean edition); sections 배경, 심층 분석

What the method computes (the pages give prose only, no formula):
  * the sequence is processed segment by segment; only the active segment
    is differentiable, history KV is detached from the graph ([FR] Contexte,
    Analyse approfondie; [JA] 背景と概要);
  * history is kept as blocks with resident per-block summaries ([JA]
    深掘り分析 on the resident block summaries that grow with length);
  * for each query block, attention runs over a bounded, exact set of
    history tokens instead of the full history, together with the active
    segment ([JA] 背景と概要; [FR] Contexte: targeted loading of a bounded
    set of relevant history tokens per query block).
The pages name resident block summaries and a bounded top-k set but define
neither, and say nothing of how a block is scored or how ties break.  The
rule below is therefore not a reading of any passage: it is the
specification this library implements, fixed outside the pages and stated
again in the C interface's header: summary = mean of the
block's keys per KV head, score = dot product with the query block's mean
query, top-k ties go to the lower block index.

Readings where the pages are silent:
  * one selection per (sequence, KV head, query block); the query mean
    averages the block's tokens and the query heads that share the KV head;
  * history = whole blocks before the segment start t0; blocks of the active
    segment are covered by the causal local part, never selected;
  * when k >= number of history blocks, every history block is taken;
  * selected indices are emitted in ascending order, padded with -1;
  * one joint softmax over selected history tokens and the causal local
    tokens, scale 1/sqrt(D); LSE in natural log;
  * gradients are truncated: dK/dV come only from queries of the same
    segment, selection receives no gradient.

Arrays: q, do [B,Hq,S,D]; k, v [B,Hkv,S,D]; query head h uses KV head
h // G with G = Hq // Hkv.  Inputs are float arrays (already rounded to the
storage dtype); everything is computed in float64.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def softmax_scale(head_dim: int, scale: Optional[float] = None) -> float:
    """Softmax temperature: 1/sqrt(D) unless given (reading; pages silent)."""
    return 1.0 / math.sqrt(head_dim) if scale is None or scale <= 0 else float(scale)


# --------------------------------------------------------------------------
# a1: resident block summaries ([JA] 深掘り分析; the mean-key reading above)
# --------------------------------------------------------------------------
def block_summaries(k: np.ndarray, hist_block: int) -> np.ndarray:
    """Mean key of every whole block: [B,Hkv,S,D] -> [B,Hkv,S//Bh,D]."""
    B, H, S, D = k.shape
    nblk = S // hist_block
    kb = _f64(k[:, :, : nblk * hist_block]).reshape(B, H, nblk, hist_block, D)
    return kb.mean(axis=3)


# --------------------------------------------------------------------------
# a2: query-block mean query (reading: one mean per KV-head group)
# --------------------------------------------------------------------------
def query_means(q: np.ndarray, n_kv_heads: int, seg_start: int, seg_len: int,
                query_block: int) -> np.ndarray:
    """Mean query of each query block of the segment, averaged over the
    query heads that share a KV head: -> [B,Hkv,nqb,D]."""
    B, Hq, S, D = q.shape
    G = Hq // n_kv_heads
    nqb = seg_len // query_block
    qs = _f64(q[:, :, seg_start:seg_start + seg_len])
    qs = qs.reshape(B, n_kv_heads, G, nqb, query_block, D)
    return qs.mean(axis=(2, 4))


# --------------------------------------------------------------------------
# a3: score + top-k ([JA] 背景と概要, [FR] Contexte; the tie reading above)
# --------------------------------------------------------------------------
def block_scores(qbar: np.ndarray, kbar: np.ndarray, nb: int,
                 precision: str = "f64") -> np.ndarray:
    """score[b,g,j,i] = qbar[b,g,j] . kbar[b,g,i] for i < nb (unscaled)."""
    if precision == "f32":
        a = np.asarray(qbar, dtype=np.float32)
        c = np.asarray(kbar[:, :, :nb], dtype=np.float32)
        return np.einsum("bgjd,bgid->bgji", a, c).astype(np.float64)
    return np.einsum("bgjd,bgid->bgji", _f64(qbar), _f64(kbar[:, :, :nb]))


def topk_blocks(scores: np.ndarray, top_k: int) -> np.ndarray:
    """Top-k of one score row: rank by (score desc, index asc), keep the
    first k, emit ascending and padded with -1 to length k."""
    nb = scores.shape[0]
    out = np.full(top_k, -1, dtype=np.int32)
    if nb <= top_k:
        out[:nb] = np.arange(nb, dtype=np.int32)
        return out
    idx = np.arange(nb)
    order = np.lexsort((idx, -scores))
    out[:] = np.sort(order[:top_k]).astype(np.int32)
    return out


def select_segment(q, k, shape, seg: int, precision: str = "f64",
                   kbar: Optional[np.ndarray] = None) -> np.ndarray:
    """Selection for every (b, g, query block) of segment `seg`:
    -> int32 [B,Hkv,nqb,k]."""
    L, Bq, Bh = shape.seg_len, shape.query_block, shape.hist_block
    t0 = seg * L
    nb = t0 // Bh
    if kbar is None:
        kbar = block_summaries(k[:, :, :t0], Bh) if nb > 0 else None
    qbar = query_means(q, shape.n_kv_heads, t0, L, Bq)
    B, Hkv, nqb, _ = qbar.shape
    sel = np.full((B, Hkv, nqb, shape.top_k), -1, dtype=np.int32)
    if nb == 0:
        return sel
    sc = block_scores(qbar, kbar, nb, precision)
    for b in range(B):
        for g in range(Hkv):
            for j in range(nqb):
                sel[b, g, j] = topk_blocks(sc[b, g, j], shape.top_k)
    return sel


def selection_gap(q, k, shape, seg: int, kbar: Optional[np.ndarray] = None) -> float:
    """Smallest score gap at the k-th boundary over the segment's query
    blocks: min over (b, g, j) of (k-th largest score) - ((k+1)-th largest
    score), where equal scores count separately (so a tie across the
    boundary gives 0).  inf when every history block is taken (nb <= k).
    Scores in fp64 from the dtype-rounded inputs.  `kbar`, when given, holds
    the summaries of at least the segment's history blocks."""
    L, Bq, Bh, kk = shape.seg_len, shape.query_block, shape.hist_block, shape.top_k
    t0 = seg * L
    nb = t0 // Bh
    if nb <= kk:
        return math.inf
    if kbar is None:
        kbar = block_summaries(k[:, :, :t0], Bh)
    qbar = query_means(q, shape.n_kv_heads, t0, L, Bq)
    sc = block_scores(qbar, kbar, nb)
    srt = -np.sort(-sc, axis=-1)
    return float(np.min(srt[..., kk - 1] - srt[..., kk]))


# --------------------------------------------------------------------------
# a4-a5: key set and forward ([JA] 背景と概要: attention over a bounded exact
# set of history tokens per query block, with the active segment)
# --------------------------------------------------------------------------
def key_indices(sel_row: np.ndarray, hist_block: int, seg_start: int,
                seg_len: int) -> tuple:
    """Token indices attended by a query block: the tokens of every selected
    history block (ascending), then the whole local segment.  Returns
    (indices, n_hist)."""
    blocks = sel_row[sel_row >= 0]
    hist = (blocks[:, None] * hist_block + np.arange(hist_block)[None, :]).reshape(-1)
    local = np.arange(seg_start, seg_start + seg_len)
    return np.concatenate([hist, local]).astype(np.int64), hist.size


def _block_mask(n_hist: int, seg_start: int, seg_len: int, q_pos: np.ndarray) -> np.ndarray:
    """[nq, n_hist + L] True where the key is visible to the query: every
    history token, and local tokens at or before the query (causal)."""
    local = np.arange(seg_start, seg_start + seg_len)
    vis_local = local[None, :] <= q_pos[:, None]
    vis_hist = np.ones((q_pos.size, n_hist), dtype=bool)
    return np.concatenate([vis_hist, vis_local], axis=1)


def _all_groups(B: int, Hkv: int):
    return [(b, g) for b in range(B) for g in range(Hkv)]


def segment_forward(q, k, v, sel, shape, seg: int, scale: Optional[float] = None,
                    groups=None):
    """O [B,Hq,L,D] and natural-log LSE [B,Hq,L] of segment `seg`, given
    its selection `sel` [B,Hkv,nqb,k].  `groups` (list of (b, g)) limits the
    work to those sequences / KV heads; other rows stay zero."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    L, Bq, Bh = shape.seg_len, shape.query_block, shape.hist_block
    t0 = seg * L
    sc = softmax_scale(D, scale)
    nqb = L // Bq
    O = np.zeros((B, Hq, L, D))
    LSE = np.zeros((B, Hq, L))
    for b, g in (groups if groups is not None else _all_groups(B, Hkv)):
        for j in range(nqb):
            keys, nh = key_indices(sel[b, g, j], Bh, t0, L)
            Kset = _f64(k[b, g, keys])
            Vset = _f64(v[b, g, keys])
            qpos = t0 + j * Bq + np.arange(Bq)
            mask = _block_mask(nh, t0, L, qpos)
            qrows = slice(t0 + j * Bq, t0 + (j + 1) * Bq)
            Qj = _f64(q[b, g * G:(g + 1) * G, qrows])         # [G,Bq,D]
            Z = sc * (Qj @ Kset.T)                            # [G,Bq,nk]
            Z = np.where(mask[None], Z, -np.inf)
            m = Z.max(axis=-1, keepdims=True)
            lse = m[..., 0] + np.log(np.exp(Z - m).sum(axis=-1))
            P = np.exp(Z - lse[..., None])
            O[b, g * G:(g + 1) * G, j * Bq:(j + 1) * Bq] = P @ Vset
            LSE[b, g * G:(g + 1) * G, j * Bq:(j + 1) * Bq] = lse
    return O, LSE


# --------------------------------------------------------------------------
# a6-a8: backward with history detached ([FR] Analyse approfondie: only the
# active segment's gradients are computed; [FR] Contexte: history states
# are kept out of the differentiable state)
# --------------------------------------------------------------------------
def segment_backward(q, k, v, do, sel, shape, seg: int, O=None, LSE=None,
                     scale: Optional[float] = None, groups=None):
    """dQ [B,Hq,L,D], dK and dV [B,Hkv,L,D] of segment `seg` for the loss
    sum(O * dO).  History keys receive no gradient; dK/dV of a local key sum
    the contributions of every query of the segment and every query head of
    its group."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    L, Bq, Bh = shape.seg_len, shape.query_block, shape.hist_block
    t0 = seg * L
    sc = softmax_scale(D, scale)
    nqb = L // Bq
    if O is None or LSE is None:
        O, LSE = segment_forward(q, k, v, sel, shape, seg, scale, groups)
    dQ = np.zeros((B, Hq, L, D))
    dK = np.zeros((B, Hkv, L, D))
    dV = np.zeros((B, Hkv, L, D))
    for b, g in (groups if groups is not None else _all_groups(B, Hkv)):
        for j in range(nqb):
            keys, nh = key_indices(sel[b, g, j], Bh, t0, L)
            Kset = _f64(k[b, g, keys])
            Vset = _f64(v[b, g, keys])
            qpos = t0 + j * Bq + np.arange(Bq)
            mask = _block_mask(nh, t0, L, qpos)
            hs = slice(g * G, (g + 1) * G)
            rows = slice(j * Bq, (j + 1) * Bq)
            qrows = slice(t0 + j * Bq, t0 + (j + 1) * Bq)
            Qj = _f64(q[b, hs, qrows])
            dOj = _f64(do[b, hs, qrows])
            Oj = _f64(O[b, hs, rows])
            lse = _f64(LSE[b, hs, rows])
            Z = sc * (Qj @ Kset.T)
            P = np.where(mask[None], np.exp(Z - lse[..., None]), 0.0)
            dP = dOj @ Vset.T
            delta = (dOj * Oj).sum(axis=-1)
            dS = P * (dP - delta[..., None])
            dQ[b, hs, rows] = sc * (dS @ Kset)
            dS_loc = dS[..., nh:]                             # [G,Bq,L]
            P_loc = P[..., nh:]
            dK[b, g] += sc * np.einsum("hqk,hqd->kd", dS_loc, Qj)
            dV[b, g] += np.einsum("hqk,hqd->kd", P_loc, dOj)
    return dQ, dK, dV


# --------------------------------------------------------------------------
# Exact-gradient backward ([SeCO] 提案手法: the forward keeps each chunk's KV
# as a checkpoint; the backward visits the chunks from the last one,
# rebuilds one chunk's graph at a time and yields exact gradients).  Applied
# to HGA, the history keys and values of a segment are no longer detached:
# they receive the gradient of every later query that selected their block.
# The selection itself is discrete and receives none.
# --------------------------------------------------------------------------
def backward_exact(q, k, v, do, sel_all, shape, O, LSE, scale: Optional[float] = None,
                   groups=None):
    """Full-sequence dQ [B,Hq,S,D], dK and dV [B,Hkv,S,D] of the loss
    sum(O * dO), where O [B,Hq,S,D] and LSE [B,Hq,S] come from the segment
    forward and sel_all [B,Hkv,S/Bq,k] holds every segment's selection.
    Segments are visited from the last to the first; each adds its queries'
    contributions to the K/V rows of its whole key set (selected history and
    causal local part), so that a segment's rows are complete when it is
    reached."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    L, Bq, Bh = shape.seg_len, shape.query_block, shape.hist_block
    sc = softmax_scale(D, scale)
    nqb = L // Bq
    dQ = np.zeros((B, Hq, S, D))
    dK = np.zeros((B, Hkv, S, D))
    dV = np.zeros((B, Hkv, S, D))
    for s in reversed(range(S // L)):
        t0 = s * L
        for b, g in (groups if groups is not None else _all_groups(B, Hkv)):
            for j in range(nqb):
                keys, nh = key_indices(sel_all[b, g, s * nqb + j], Bh, t0, L)
                Kset = _f64(k[b, g, keys])
                Vset = _f64(v[b, g, keys])
                qpos = t0 + j * Bq + np.arange(Bq)
                mask = _block_mask(nh, t0, L, qpos)
                hs = slice(g * G, (g + 1) * G)
                qrows = slice(t0 + j * Bq, t0 + (j + 1) * Bq)
                Qj = _f64(q[b, hs, qrows])
                dOj = _f64(do[b, hs, qrows])
                lse = _f64(LSE[b, hs, qrows])
                Z = sc * (Qj @ Kset.T)
                P = np.where(mask[None], np.exp(Z - lse[..., None]), 0.0)
                dP = dOj @ Vset.T
                delta = (dOj * _f64(O[b, hs, qrows])).sum(axis=-1)
                dS = P * (dP - delta[..., None])
                dQ[b, hs, qrows] = sc * (dS @ Kset)
                # keys are distinct within one key set, so plain indexed adds
                dK[b, g, keys] += sc * np.einsum("hqk,hqd->kd", dS, Qj)
                dV[b, g, keys] += np.einsum("hqk,hqd->kd", P, dOj)
    return dQ, dK, dV


# --------------------------------------------------------------------------
# a9: the segment loop ([FR] Analyse approfondie: the input is processed in
# segments, one after another)
# --------------------------------------------------------------------------
def run(inputs: dict, shape=None, segments=None, bwd: Optional[bool] = None,
        precision: str = "f64", scale: Optional[float] = None) -> dict:
    """Whole segmented pass (or the listed segments).  Returns full-sequence
    arrays: kbar [B,Hkv,S//Bh,D], sel [B,Hkv,S//Bq,k], o, lse, and if bwd:
    dq, dk, dv.  Rows of segments not listed stay zero (sel: -1)."""
    shape = shape or inputs["shape"]
    q, k, v, do = inputs["q"], inputs["k"], inputs["v"], inputs.get("do")
    if bwd is None:
        bwd = shape.bwd and do is not None
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    L, Bq = shape.seg_len, shape.query_block
    segments = range(S // L) if segments is None else segments
    nqb = L // Bq
    out = {
        "kbar": block_summaries(k, shape.hist_block),
        "sel": np.full((B, Hkv, S // Bq, shape.top_k), -1, dtype=np.int32),
        "o": np.zeros((B, Hq, S, D)),
        "lse": np.zeros((B, Hq, S)),
    }
    if bwd:
        out["dq"] = np.zeros((B, Hq, S, D))
        out["dk"] = np.zeros((B, Hkv, S, D))
        out["dv"] = np.zeros((B, Hkv, S, D))
    for s in segments:
        t0 = s * L
        sel = select_segment(q, k, shape, s, precision,
                             kbar=out["kbar"] if t0 > 0 else None)
        out["sel"][:, :, s * nqb:(s + 1) * nqb] = sel
        O, LSE = segment_forward(q, k, v, sel, shape, s, scale)
        out["o"][:, :, t0:t0 + L] = O
        out["lse"][:, :, t0:t0 + L] = LSE
        if bwd:
            dQ, dK, dV = segment_backward(q, k, v, do, sel, shape, s, O, LSE, scale)
            out["dq"][:, :, t0:t0 + L] = dQ
            out["dk"][:, :, t0:t0 + L] = dK
            out["dv"][:, :, t0:t0 + L] = dV
    return out


def gather_blocks(x: np.ndarray, sel: np.ndarray, hist_block: int) -> np.ndarray:
    """a4 as a standalone copy: for sel [B,Hkv,nqb,k] return the chosen
    blocks of x [B,Hkv,S,D] as [B,Hkv,nqb,k,Bh,D]; padded slots are zero.
    Values are copied unchanged (no arithmetic)."""
    B, H, nqb, kk = sel.shape
    D = x.shape[-1]
    out = np.zeros((B, H, nqb, kk, hist_block, D), dtype=x.dtype)
    for b in range(B):
        for g in range(H):
            for j in range(nqb):
                for t in range(kk):
                    blk = sel[b, g, j, t]
                    if blk >= 0:
                        out[b, g, j, t] = x[b, g, blk * hist_block:(blk + 1) * hist_block]
    return out


# --------------------------------------------------------------------------
# Decode step ([JA] 深掘り分析: after training, inference runs over sequences
# of up to 131,072 tokens while the resident block summaries grow; [JA]
# 業界への影響 and [FR] Contexte: HGA as a module for retrieval and
# generation).  The pages describe no decode procedure; the reading here is
# the forward above applied to a query block made of the new tokens.
# --------------------------------------------------------------------------
def decode_step(q_new, k, v, shape, pos: int, scale: Optional[float] = None,
                precision: str = "f64", kbar: Optional[np.ndarray] = None):
    """One step for n new tokens at positions pos .. pos+n-1, all inside one
    segment.  q_new [B,Hq,n,D]; k, v [B,Hkv,S,D] hold every token up to
    pos+n-1.  Readings (pages silent):
      * the new tokens form one query block of the segment that holds them,
        t0 = floor(pos / L) * L; history = the whole blocks before t0;
      * selection as for a segment's query block: qbar = mean of q_new over
        the G heads of the group and the n tokens, score = qbar . kbar,
        top-k by (score desc, index asc), ascending, -1 padded;
      * token pos+i attends to the selected history tokens and the local
        tokens t0 .. pos+i with one joint softmax.
    Returns (sel [B,Hkv,k] int32, O [B,Hq,n,D], LSE [B,Hq,n])."""
    B, Hq, n, D = q_new.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    L, Bh, kk = shape.seg_len, shape.hist_block, shape.top_k
    t0 = (pos // L) * L
    if n < 1 or (pos + n - 1) // L != pos // L:
        raise ValueError("the new tokens must lie inside one segment")
    nb = t0 // Bh
    sc = softmax_scale(D, scale)
    sel = np.full((B, Hkv, kk), -1, dtype=np.int32)
    if nb > 0:
        if kbar is None:
            kbar = block_summaries(k[:, :, :t0], Bh)
        qbar = _f64(q_new).reshape(B, Hkv, G, n, D).mean(axis=(2, 3))[:, :, None]
        scores = block_scores(qbar, kbar, nb, precision)[:, :, 0]   # [B,Hkv,nb]
        for b in range(B):
            for g in range(Hkv):
                sel[b, g] = topk_blocks(scores[b, g], kk)
    O = np.zeros((B, Hq, n, D))
    LSE = np.zeros((B, Hq, n))
    qpos = pos + np.arange(n)
    nloc = pos + n - t0
    for b in range(B):
        for g in range(Hkv):
            blocks = sel[b, g][sel[b, g] >= 0]
            hist = (blocks[:, None] * Bh + np.arange(Bh)[None, :]).reshape(-1)
            keys = np.concatenate([hist, np.arange(t0, t0 + nloc)]).astype(np.int64)
            vis = np.concatenate([np.ones((n, hist.size), dtype=bool),
                                  np.arange(t0, t0 + nloc)[None, :] <= qpos[:, None]], axis=1)
            Kset = _f64(k[b, g, keys])
            Vset = _f64(v[b, g, keys])
            Qg = _f64(q_new[b, g * G:(g + 1) * G])                 # [G,n,D]
            Z = np.where(vis[None], sc * (Qg @ Kset.T), -np.inf)
            m = Z.max(axis=-1, keepdims=True)
            lse = m[..., 0] + np.log(np.exp(Z - m).sum(axis=-1))
            O[b, g * G:(g + 1) * G] = np.exp(Z - lse[..., None]) @ Vset
            LSE[b, g * G:(g + 1) * G] = lse
    return sel, O, LSE
