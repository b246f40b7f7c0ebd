"""Pins of the oracle's exact-gradient backward (history not detached)
against torch float64 autograd, which differentiates the same attention
without any of the oracle's bookkeeping: (1) with k covering the history,
the gradients of dense causal attention over the whole sequence; (2) for
any k, the gradients of full-sequence attention under the boolean mask that
the selection implies.  A planted mistake in the reverse-order accumulation
(a history row dropped, a contribution added twice) fails (2)."""

import numpy as np
import pytest
import torch

from oracle import hga_oracle as orc
from synth import HGAShape, make_inputs


def shp(**kw):
    base = dict(name="x", batch=1, seq_len=64, n_q_heads=2, n_kv_heads=1, head_dim=8,
                seg_len=16, hist_block=8, query_block=8, top_k=2, dtype="f32")
    base.update(kw)
    return HGAShape(**base)


def _oracle_exact(inp, shape):
    out = orc.run(inp, shape, bwd=False)
    return orc.backward_exact(inp["q"], inp["k"], inp["v"], inp["do"], out["sel"], shape,
                              out["o"], out["lse"]), out


def _torch_grads(inp, shape, mask):
    """float64 autograd of sum(SDPA(q, k, v; mask) * dO) over the whole
    sequence, GQA by repeat_interleave (gradients flow back to k, v)."""
    G = shape.group
    q = torch.tensor(inp["q"], dtype=torch.float64, requires_grad=True)
    k = torch.tensor(inp["k"], dtype=torch.float64, requires_grad=True)
    v = torch.tensor(inp["v"], dtype=torch.float64, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1),
        attn_mask=torch.as_tensor(mask))
    (o * torch.tensor(inp["do"], dtype=torch.float64)).sum().backward()
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _full_mask(sel, shape):
    """[B,Hq,S,S] visibility: each query sees the tokens of the blocks
    selected for its (KV head, query block) and its segment's tokens up to
    itself."""
    B, Hq, S = shape.batch, shape.n_q_heads, shape.seq_len
    L, Bq, Bh, G = shape.seg_len, shape.query_block, shape.hist_block, shape.group
    m = np.zeros((B, Hq, S, S), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            for t in range(S):
                t0 = t // L * L
                for blk in sel[b, h // G, t // Bq]:
                    if blk >= 0:
                        m[b, h, t, blk * Bh:(blk + 1) * Bh] = True
                m[b, h, t, t0:t + 1] = True
    return m


@pytest.mark.parametrize("shape", [
    shp(top_k=8),                                                         # k covers all
    shp(n_q_heads=4, n_kv_heads=2, seq_len=96, seg_len=32, hist_block=16, top_k=5),
])
def test_exact_equals_dense_causal_when_k_covers_history(shape):
    inp = make_inputs(shape, seed=4)
    (dQ, dK, dV), out = _oracle_exact(inp, shape)
    S = shape.seq_len
    causal = np.tril(np.ones((S, S), dtype=bool))
    o, gq, gk, gv = _torch_grads(inp, shape, np.broadcast_to(causal, (1, 1, S, S)).copy())
    np.testing.assert_allclose(out["o"], o, rtol=0, atol=1e-12)
    for name, x, ref in (("dq", dQ, gq), ("dk", dK, gk), ("dv", dV, gv)):
        np.testing.assert_allclose(x, ref, rtol=0, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("shape", [
    shp(),
    shp(n_q_heads=4, n_kv_heads=2, seq_len=96, seg_len=32, hist_block=16, query_block=8,
        top_k=3, head_dim=16),
    shp(batch=2, hist_block=4, query_block=16, top_k=5),
])
def test_exact_matches_torch_autograd_under_the_selection_mask(shape):
    inp = make_inputs(shape, seed=17)
    (dQ, dK, dV), out = _oracle_exact(inp, shape)
    o, gq, gk, gv = _torch_grads(inp, shape, _full_mask(out["sel"], shape))
    np.testing.assert_allclose(out["o"], o, rtol=0, atol=1e-12)
    for name, x, ref in (("dq", dQ, gq), ("dk", dK, gk), ("dv", dV, gv)):
        np.testing.assert_allclose(x, ref, rtol=0, atol=1e-11, err_msg=name)


def test_exact_local_rows_differ_from_truncated_only_by_history_terms():
    """dQ is the same as the truncated backward's; dK/dV of the last
    segment (no later query can select it) are the same too."""
    shape = shp(top_k=3)
    inp = make_inputs(shape, seed=8)
    (dQ, dK, dV), _ = _oracle_exact(inp, shape)
    tr = orc.run(inp, shape, bwd=True)
    np.testing.assert_allclose(dQ, tr["dq"], rtol=0, atol=1e-12)
    last = slice(shape.seq_len - shape.seg_len, shape.seq_len)
    np.testing.assert_allclose(dK[:, :, last], tr["dk"][:, :, last], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV[:, :, last], tr["dv"][:, :, last], rtol=0, atol=1e-12)
    assert np.abs(dK[:, :, :shape.seg_len] - tr["dk"][:, :, :shape.seg_len]).max() > 1e-3
