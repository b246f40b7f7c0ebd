"""Planted-direction N(0,1) generator for HGA workloads.

Page keys used in citations (the pages are news write-ups of one method):
  [JA] 「低VRAM長文脈ファインチューニング：階層的グローバル注意と分割バック
       プロpagationの実践」, sns.style (Japanese edition)
  [FR] « Ajustement fin long-contexte à faible VRAM : une approche
       d'optimisation avec attention globale hiérarchique », sns.style

The pages benchmark on PG19 with Qwen3-8B activations ([JA] 深掘り分析).
Neither is available, so seeded synthetic tensors of the same attention
shape (32 query heads sharing 8 KV heads, head_dim 128) stand in.  Kernel
cost depends only on shapes and on which history blocks get selected, never
on token content, so a generator that controls selection is enough.

Recipe (per sequence b, with seed_b = seed + b):
  1. One ``numpy.random.SeedSequence(seed_b)`` spawns six independent
     streams: Q, K, V, dO, directions, planting.  Independent streams let a
     forward-only workload skip dO without changing Q/K/V.
  2. Q [Hq,S,D], K [Hkv,S,D], V [Hkv,S,D], dO [Hq,S,D] ~ N(0,1) float32.
  3. Directions: QR of a D x (nseg-1) Gaussian matrix, columns sign-fixed so
     that diag(R) > 0, giving mutually orthogonal unit vectors u_1..u_{nseg-1}
     (when nseg-1 > D, plain normalised Gaussian vectors instead).
  4. For every segment s >= 1 with nb = s*L/Bh history blocks:
     choose min(k, nb) distinct earlier blocks (sorted), add 2*u_s to every
     query of segment s (all query heads) and to every key of the chosen
     blocks (all KV heads).  The chosen blocks are therefore the ones whose
     mean key points along the segment's mean query.
  5. Round all tensors to the storage dtype (bf16: round to nearest even),
     and keep them as float32 arrays holding exactly representable values.

"Diverse" mode (throughput variant) plants one direction per (segment,
query block) instead of one per segment, so query blocks of one segment
pick different history sets; its directions are not orthogonal.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class HGAShape:
    """Problem shape of one HGA layer over one batch of sequences."""

    name: str
    batch: int
    seq_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seg_len: int
    hist_block: int
    query_block: int
    top_k: int
    dtype: str  # "f32" or "bf16"
    bwd: bool = True

    @property
    def nseg(self) -> int:
        return self.seq_len // self.seg_len

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_qblocks(self) -> int:
        return self.seg_len // self.query_block

    def n_hist_blocks(self, seg: int) -> int:
        return (seg * self.seg_len) // self.hist_block

    def replace(self, **kw) -> "HGAShape":
        return dataclasses.replace(self, **kw)

    def validate(self) -> None:
        assert self.seq_len % self.seg_len == 0
        assert self.seg_len % self.hist_block == 0
        assert self.seg_len % self.query_block == 0
        assert self.n_q_heads % self.n_kv_heads == 0
        assert self.top_k >= 1


# The five workloads the method is measured on.  Shapes follow the pages'
# model (Qwen3-8B attention: 32 query heads, 8 KV heads, head_dim 128;
# [JA] 深掘り分析), the 16,384-token training length and the 131,072-token
# inference length ([JA] 深掘り分析).
WORKLOADS: Dict[str, HGAShape] = {
    s.name: s
    for s in [
        HGAShape("tiny_f32", 1, 512, 2, 1, 64, 128, 32, 32, 4, "f32"),
        HGAShape("qwen3_2k", 1, 2048, 32, 8, 128, 512, 64, 64, 8, "bf16"),
        HGAShape("train_16k", 1, 16384, 32, 8, 128, 1024, 64, 64, 32, "bf16"),
        HGAShape("infer_131k", 1, 131072, 32, 8, 128, 1024, 128, 128, 16,
                 "bf16", bwd=False),
        HGAShape("batch4_32k", 4, 32768, 32, 8, 128, 2048, 128, 128, 16,
                 "bf16"),
    ]
}


def shape_by_name(name: str) -> HGAShape:
    return WORKLOADS[name]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values in place to the nearest bf16 (ties to even).

    Works in chunks along the first axis to bound temporary memory.
    Returns the same array, whose values are now exactly bf16-representable.
    """
    assert x.dtype == np.float32 and x.flags.c_contiguous
    flat = x.reshape(x.shape[0], -1) if x.ndim > 1 else x.reshape(1, -1)
    for row in range(flat.shape[0]):
        bits = flat[row].view(np.uint32)
        lsb = (bits >> np.uint32(16)) & np.uint32(1)
        bits += np.uint32(0x7FFF) + lsb
        bits &= np.uint32(0xFFFF0000)
    return x


def _directions(rng: np.random.Generator, dim: int, count: int) -> np.ndarray:
    """`count` unit vectors of length `dim` as columns (orthogonal if possible)."""
    if count == 0:
        return np.zeros((dim, 0), dtype=np.float64)
    g = rng.standard_normal((dim, count))
    if count <= dim:
        qm, rm = np.linalg.qr(g)
        signs = np.sign(np.diag(rm))
        signs[signs == 0] = 1.0
        return qm * signs[None, :]
    return g / np.linalg.norm(g, axis=0, keepdims=True)


def make_inputs(shape: HGAShape, seed: int = 0, with_do: Optional[bool] = None,
                mode: str = "planted", amplitude: float = 2.0) -> dict:
    """Draw Q, K, V (and dO) for `shape`.

    Returns a dict with float32 arrays ``q`` [B,Hq,S,D], ``k``/``v``
    [B,Hkv,S,D], ``do`` [B,Hq,S,D] or None, plus ``planted``: for each
    sequence, for each segment, the sorted array of planted block indices
    (for diverse mode: one array per (segment, query block)).
    """
    shape.validate()
    if with_do is None:
        with_do = shape.bwd
    B, S, D = shape.batch, shape.seq_len, shape.head_dim
    Hq, Hkv = shape.n_q_heads, shape.n_kv_heads
    L, Bh, Bq, k = shape.seg_len, shape.hist_block, shape.query_block, shape.top_k
    nseg = shape.nseg

    q = np.empty((B, Hq, S, D), dtype=np.float32)
    kk = np.empty((B, Hkv, S, D), dtype=np.float32)
    v = np.empty((B, Hkv, S, D), dtype=np.float32)
    do = np.empty((B, Hq, S, D), dtype=np.float32) if with_do else None
    planted: List[list] = []

    for b in range(B):
        ss = np.random.SeedSequence(seed + b)
        s_q, s_k, s_v, s_do, s_dir, s_plant = ss.spawn(6)
        np.random.default_rng(s_q).standard_normal(out=q[b], dtype=np.float32)
        np.random.default_rng(s_k).standard_normal(out=kk[b], dtype=np.float32)
        np.random.default_rng(s_v).standard_normal(out=v[b], dtype=np.float32)
        if with_do:
            np.random.default_rng(s_do).standard_normal(out=do[b], dtype=np.float32)
        rng_dir = np.random.default_rng(s_dir)
        rng_plant = np.random.default_rng(s_plant)
        per_seq: list = [np.zeros(0, dtype=np.int64)]
        if mode == "planted":
            dirs = _directions(rng_dir, D, nseg - 1)
            for s in range(1, nseg):
                nb = shape.n_hist_blocks(s)
                chosen = np.sort(rng_plant.choice(nb, size=min(k, nb), replace=False))
                u = (amplitude * dirs[:, s - 1]).astype(np.float32)
                t0 = s * L
                q[b, :, t0:t0 + L, :] += u
                for blk in chosen:
                    kk[b, :, blk * Bh:(blk + 1) * Bh, :] += u
                per_seq.append(chosen)
        elif mode == "diverse":
            nqb = shape.n_qblocks
            dirs = _directions(rng_dir, D, max(0, (nseg - 1) * nqb))
            per_seq = [[np.zeros(0, dtype=np.int64)] * nqb]
            for s in range(1, nseg):
                nb = shape.n_hist_blocks(s)
                t0 = s * L
                row = []
                for j in range(nqb):
                    chosen = np.sort(rng_plant.choice(nb, size=min(k, nb), replace=False))
                    u = (amplitude * dirs[:, (s - 1) * nqb + j]).astype(np.float32)
                    q[b, :, t0 + j * Bq:t0 + (j + 1) * Bq, :] += u
                    for blk in chosen:
                        kk[b, :, blk * Bh:(blk + 1) * Bh, :] += u
                    row.append(chosen)
                per_seq.append(row)
        else:
            raise ValueError(f"unknown mode {mode!r}")
        planted.append(per_seq)

    if shape.dtype == "bf16":
        for arr in (q, kk, v, do):
            if arr is not None:
                round_to_bf16(arr)
    elif shape.dtype != "f32":
        raise ValueError(f"unknown dtype {shape.dtype!r}")

    return {"q": q, "k": kk, "v": v, "do": do, "planted": planted,
            "seed": seed, "mode": mode, "shape": shape}

