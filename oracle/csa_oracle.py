"""CPU reference (oracle) for the compressed-sparse-attention decode path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run this module; the library
and its Python binding never do, and there is no CPU fallback anywhere in the
product path.

Plain, slow, fp64 numpy.  It shares no code with the HIP path: it decodes the
bf16 inputs itself, computes every quantity from its definition, and uses only
library primitives (matrix product, sort, exp/log) as single steps.

Sources (web pages of the ``nvfp4-megamoe-kernel`` design notes):

* [P1] "ARCHITECTURE & MEMORY AUDIT -- Post-probe rewrite": F1 (indexer keys are
  one ``c_I``-wide vector per compressed block shared by all indexer heads),
  F3 (the scoring formula, eq. 16 of DeepSeek-V4 sec. 2.3.1 as restated there,
  and the corrected einsum / top-k), B1-B2 (concatenate the selected compressed
  rows with the SWA rows), C2 (gather into one preallocated buffer).
* [P2] "ARCHITECTURE & MEMORY AUDIT -- 1M-context viability": D3 (gather then
  concat), D4 (HCA attends over the entire compressed history plus SWA),
  D5 (FMHA input = selected compressed ++ sliding window), D6 (attention sink =
  a per-head additive logit in the softmax denominator).
* [P3] "PART A -- Next Session Clues": suspect 3 (a decode query sees only
  compressed blocks strictly before its own, incomplete block; the newest
  tokens are attended both in SWA and in the newest compressed block).

Readings where the pages are silent:

* visible blocks of a query at 0-based position ``pos`` = ``floor(pos/ratio)``,
  capped by the blocks stored for its sequence;
* ties at the k-th score go to the lower block index (any tied choice is an
  equally valid selection; the GPU is checked against the tie band, not this
  order);
* fewer visible blocks than ``top_k`` selects all of them; none selected means
  SWA-only attention;
* keys and values of the shared-KV attention are the same row; the softmax scale
  is an argument; an empty row set gives a zero output and ``lse = -inf``.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64.  bf16 is the top half
    of an IEEE float32, so the value is exact in float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def visible_blocks(pos: int, ratio: int, n_comp: int) -> int:
    """Number of compressed blocks a query at 0-based position ``pos`` may see.

    [P3] suspect 3: only blocks strictly preceding the query's own (incomplete)
    block are visible.  Block b covers positions [b*ratio, (b+1)*ratio); the
    query's own block is floor(pos/ratio), so blocks 0..floor(pos/ratio)-1 are
    visible -- never more than the sequence has stored.
    """
    if pos < 0 or ratio <= 0:
        raise ValueError("pos must be >= 0 and ratio > 0")
    return int(min(pos // ratio, n_comp))


def indexer_scores(q_idx: np.ndarray, w: np.ndarray, keys: np.ndarray):
    """Lightning-indexer scores of one query token against ``keys``.

    [P1] F3, eq. 16 (DeepSeek-V4 sec. 2.3.1 as restated there):
        I[s] = sum_h  w[h] * ReLU( q_idx[h] . K[s] )
    with ONE key per block shared by every indexer head ([P1] F1: keys carry no
    head axis; the per-head-key form is the refuted algebra).

    q_idx: [n_ih, ihd] float64; w: [n_ih]; keys: [n, ihd].
    Returns (I, A): I[s] the score, A[s] = sum_h |w[h]| * ReLU(q_idx[h].K[s]),
    the magnitude scale used to state a tolerance for a rounded computation.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(0), np.zeros(0)
    logits = keys @ q_idx.T                  # [n, n_ih]: q_idx[h] . K[s]
    relu = np.maximum(logits, 0.0)           # ReLU per head
    return relu @ w, relu @ np.abs(w)        # weighted sum over heads


def select_top_blocks(I: np.ndarray, top_k: int) -> np.ndarray:
    """Indices of the ``min(top_k, len(I))`` largest scores.

    [P1] F3: ``tk = min(top_k, n_comp)`` then ``total.topk(tk)``; here applied to
    the visible scores only ([P3] suspect 3).  Returned in descending score
    order; equal scores are taken lowest index first.
    """
    I = np.asarray(I, dtype=np.float64)
    n = I.shape[0]
    k_eff = min(int(top_k), n)
    if k_eff <= 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((np.arange(n), -I))   # primary: -I ascending; then index
    return order[:k_eff].astype(np.int64)


def gather_rows(comp_kv: np.ndarray, sel: np.ndarray, swa_rows: np.ndarray) -> np.ndarray:
    """Attention row set of one CSA query: the selected compressed rows, then
    the sliding-window rows.

    [P1] B1/B2 and [P2] D3/D5: ``all_kv = cat(comp_kv[topk], swa_kv)``; [P1] C2
    writes the selected rows first and the SWA rows right after them.  No
    de-duplication of tokens present in both ([P3] suspect 3).
    """
    sel = np.asarray(sel, dtype=np.int64)
    return np.concatenate([np.asarray(comp_kv)[sel], np.asarray(swa_rows)], axis=0)


def shared_kv_attention(q: np.ndarray, rows: np.ndarray, scale: float,
                        sink: Optional[np.ndarray] = None):
    """Softmax attention of every head of ``q`` over one shared set of rows.

    [P1] F3 / [P2] D6 ("shared key-value MQA", DeepSeek-V4 sec. 2.3.1): each row
    is both the key and the value, shared by all query heads.  Per head h:
        z_j = scale * q[h] . row_j
        o_h = sum_j exp(z_j) row_j / (sum_j exp(z_j) + exp(sink_h))
    where the sink term ([P2] D6: a per-head additive logit in the denominator)
    is present only when ``sink`` is given.  Also returns
    lse_h = log(sum_j exp(z_j) + exp(sink_h)).
    q: [H, D]; rows: [n, D].  n == 0 (and no sink) gives zeros and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    H, D = q.shape
    n = rows.shape[0]
    if n == 0 and sink is None:
        return np.zeros((H, D)), np.full(H, -np.inf)
    z = scale * (q @ rows.T)                                  # [H, n]
    m = z.max(axis=1) if n else np.full(H, -np.inf)
    if sink is not None:
        m = np.maximum(m, np.asarray(sink, dtype=np.float64))
    p = np.exp(z - m[:, None])
    Z = p.sum(axis=1)
    if sink is not None:
        Z = Z + np.exp(np.asarray(sink, dtype=np.float64) - m)
    out = (p @ rows) / Z[:, None]
    return out, m + np.log(Z)


def csa_token(inp, t: int, sink: Optional[np.ndarray] = None) -> dict:
    """The whole CSA decode path for query token ``t`` of a CSAInputs batch:
    visibility -> indexer scores -> top-k -> gather -> shared-KV attention."""
    row0 = int(inp.seq_kv[t])
    n_vis = visible_blocks(int(inp.pos[t]), inp.ratio, int(inp.n_comp[t]))
    keys = bf16_to_f64(inp.k_idx[row0:row0 + n_vis])
    I, A = indexer_scores(bf16_to_f64(inp.q_idx[t]), inp.w[t], keys)
    sel = select_top_blocks(I, inp.top_k)
    s0, sl = int(inp.swa_row0[t]), int(inp.swa_len[t])
    comp = inp.comp_kv[row0:row0 + n_vis]
    rows_bits = gather_rows(comp, sel, inp.swa[s0:s0 + sl])
    out, lse = shared_kv_attention(bf16_to_f64(inp.q[t]), bf16_to_f64(rows_bits),
                                   inp.scale, sink)
    return dict(n_vis=n_vis, scores=I, scale_A=A, sel=sel, rows=rows_bits,
                out=out, lse=lse)


def hca_token(q: np.ndarray, comp_kv: np.ndarray, n_vis: int, swa_rows: np.ndarray,
              scale: float, sink: Optional[np.ndarray] = None):
    """Dense HCA query: attention over the entire visible compressed history
    followed by the SWA rows, no indexer ([P2] D4)."""
    rows = np.concatenate([np.asarray(comp_kv)[:n_vis], np.asarray(swa_rows)], axis=0)
    return shared_kv_attention(bf16_to_f64(q), bf16_to_f64(rows), scale, sink)
