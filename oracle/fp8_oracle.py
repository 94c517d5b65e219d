"""CPU reference for the FP8 indexer keys and queries (test infrastructure
only, like the rest of ``oracle/``: never imported by the library or its
binding).

[P1] "ARCHITECTURE & MEMORY AUDIT -- Post-probe rewrite", C4, and [P2]
"ARCHITECTURE & MEMORY AUDIT -- 1M-context viability", M1/A2: the indexer's
keys (and query activations) are meant to be stored and multiplied in a
narrow floating-point format, the storage paired with a low-precision
scoring product, and gated on top-k recall against a full-precision oracle
(>= 99.7 % at top_k 1024).  The pages name FP4; this build uses the OCP FP8
E4M3 ("E4M3FN") format, the one gfx950's FP8 matrix instructions read.

Readings where the pages are silent (plain, exactly reproducible choices):

* one power-of-two scale per row (per key block, or per query token and
  head): the smallest ``2**e`` with ``max|x| * 2**-e <= 448`` (448 is E4M3's
  largest finite value); ``e = 0`` for an all-zero row.  A power of two
  scales exactly, so the quantised codes are a function of the inputs alone;
* each element ``x * 2**-e`` is rounded to the nearest E4M3 value, ties to
  even, including the subnormals (spacing 2**-9); no value exceeds 448 by
  construction of the scale;
* the scores of quantised inputs are the indexer scores of the dequantised
  inputs (``code value * 2**e``): the method's formula, unchanged.
"""
from __future__ import annotations

import math

import numpy as np

from .csa_oracle import (bf16_to_f64, gather_rows, indexer_scores, select_top_blocks,
                         shared_kv_attention, visible_blocks)

E4M3_MAX = 448.0


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 bytes: sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 is subnormal (m/8 * 2**-6); S.1111.111 is NaN (the
    format has no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _round_e4m3(y: float) -> int:
    """E4M3 code of the real y (|y| <= 448): nearest value, ties to even."""
    if math.isnan(y) or abs(y) > E4M3_MAX:
        raise ValueError("outside the E4M3 range")
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    if a < 2.0 ** -6:
        # subnormal: multiples of 2**-9; 8 * 2**-9 is the smallest normal,
        # whose code (0x08) follows the subnormals'
        q = a * 2.0 ** 9
        n = math.floor(q)
        r = q - n
        if r > 0.5 or (r == 0.5 and n % 2 == 1):
            n += 1
        return sign | n
    E = math.frexp(a)[1] - 1          # a = f * 2**E, 1 <= f < 2
    f = a / 2.0 ** E
    q = (f - 1.0) * 8.0               # mantissa in eighths
    n = math.floor(q)
    r = q - n
    if r > 0.5 or (r == 0.5 and n % 2 == 1):
        n += 1
    if n == 8:
        n = 0
        E += 1
    return sign | ((E + 7) << 3) | n


def row_scale_exponent(row: np.ndarray) -> int:
    """Smallest e with max|row| * 2**-e <= 448 (0 for an all-zero row)."""
    amax = float(np.max(np.abs(row))) if row.size else 0.0
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / E4M3_MAX))
    # settle the boundary exactly (log2 is not exact)
    while amax * 2.0 ** -e > E4M3_MAX:
        e += 1
    while amax * 2.0 ** -(e - 1) <= E4M3_MAX:
        e -= 1
    return e


def quantize_rows_e4m3(x: np.ndarray):
    """Quantise every row of x (float64, last axis = row) to E4M3 with its
    own power-of-two scale.  Returns (codes uint8 of x's shape, scale float64
    of x.shape[:-1]) with x ~= e4m3_to_f64(codes) * scale[..., None].

    Vectorised form of row_scale_exponent and _round_e4m3 (the tests check
    that the two agree code for code): with amax = f * 2**E, 1 <= f < 2, the
    smallest admissible exponent is E - 8 when f <= 1.75 (448 = 1.75 * 2**8)
    and E - 7 otherwise; np.rint rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    rows = x.reshape(-1, x.shape[-1])
    amax = np.max(np.abs(rows), axis=1) if rows.shape[1] else np.zeros(rows.shape[0])
    fm, ex = np.frexp(amax)            # amax = fm * 2**ex, 0.5 <= fm < 1
    e = np.where(2.0 * fm <= 1.75, ex - 1 - 8, ex - 1 - 7)
    e = np.where(amax == 0.0, 0, e).astype(np.int64)
    y = rows * np.exp2(-e.astype(np.float64))[:, None]   # exact: a power of two
    a = np.abs(y)
    _, ey = np.frexp(np.where(a > 0, a, 1.0))
    E = ey - 1
    n = np.rint((a / np.exp2(E.astype(np.float64)) - 1.0) * 8.0)
    carry = n == 8
    n = np.where(carry, 0, n)
    E = np.where(carry, E + 1, E)
    code_norm = ((E + 7) << 3).astype(np.int64) | n.astype(np.int64)
    code_sub = np.rint(a * 512.0).astype(np.int64)
    code = np.where(a >= 2.0 ** -6, code_norm, code_sub)
    code = code | np.where(np.signbit(y), 0x80, 0)
    return (code.astype(np.uint8).reshape(x.shape),
            np.exp2(e.astype(np.float64)).reshape(x.shape[:-1]))


def quantize_rows_e4m3_scalar(x: np.ndarray):
    """The same quantisation element by element from row_scale_exponent and
    _round_e4m3 (slow; the pin for quantize_rows_e4m3)."""
    x = np.asarray(x, dtype=np.float64)
    rows = x.reshape(-1, x.shape[-1])
    codes = np.empty(rows.shape, dtype=np.uint8)
    scale = np.empty(rows.shape[0], dtype=np.float64)
    for i, row in enumerate(rows):
        e = row_scale_exponent(row)
        scale[i] = 2.0 ** e
        for j, v in enumerate(row):
            codes[i, j] = _round_e4m3(v * 2.0 ** -e)
    return codes.reshape(x.shape), scale.reshape(x.shape[:-1])


def indexer_scores_e4m3(q_codes: np.ndarray, q_scale: np.ndarray, w: np.ndarray,
                        k_codes: np.ndarray, k_scale: np.ndarray):
    """Indexer scores of one query token from E4M3 queries [n_ih, ihd] (scale
    per head) and keys [n, ihd] (scale per block): [P1] F3's formula on the
    dequantised values.  Returns (I, A) as indexer_scores does."""
    q = e4m3_to_f64(q_codes) * np.asarray(q_scale, dtype=np.float64)[:, None]
    k = e4m3_to_f64(k_codes) * np.asarray(k_scale, dtype=np.float64)[:, None]
    return indexer_scores(q, w, k)


def prefilter_count(top_k: int) -> int:
    """Candidates the E4M3 prefilter keeps: half as many again as top_k (at
    most 4096).  A reading of [P1] C4 with [P2] A2's recall gate: narrow
    products rank the blocks, and the full-precision scores of a margin of
    candidates around the top_k decide the selection."""
    return min(int(top_k) + int(top_k) // 2, 4096)


def select_prefiltered(I8: np.ndarray, I: np.ndarray, top_k: int, C: int):
    """The min(top_k, n) blocks with the largest bf16 scores I among the
    min(C, n) blocks with the largest E4M3 scores I8; both orders take the
    lower block index first on equal scores.  Returns (selection in
    descending I order, candidates in ascending block order)."""
    cand = np.sort(select_top_blocks(I8, C))
    inner = select_top_blocks(np.asarray(I, dtype=np.float64)[cand], top_k)
    return cand[inner], cand


def csa_token_e4m3(inp, t: int, sink=None) -> dict:
    """The CSA decode path for token t with the E4M3 indexer prefilter: the
    token's indexer queries and its visible keys quantised row by row, scored
    (scores8), the prefilter_count(top_k) best kept, their bf16 scores
    deciding the top_k; gather and attention as in csa_token."""
    row0 = int(inp.seq_kv[t])
    n_vis = visible_blocks(int(inp.pos[t]), inp.ratio, int(inp.n_comp[t]))
    q = bf16_to_f64(inp.q_idx[t])
    keys = bf16_to_f64(inp.k_idx[row0:row0 + n_vis])
    qc, qs = quantize_rows_e4m3(q)
    kc, ks = quantize_rows_e4m3(keys)
    I8, A8 = indexer_scores_e4m3(qc, qs, inp.w[t], kc, ks)
    I, A = indexer_scores(q, inp.w[t], keys)
    sel, cand = select_prefiltered(I8, I, inp.top_k, prefilter_count(inp.top_k))
    s0, sl = int(inp.swa_row0[t]), int(inp.swa_len[t])
    rows_bits = gather_rows(inp.comp_kv[row0:row0 + n_vis], sel, inp.swa[s0:s0 + sl])
    out, lse = shared_kv_attention(bf16_to_f64(inp.q[t]), bf16_to_f64(rows_bits), inp.scale, sink)
    return dict(n_vis=n_vis, scores8=I8, scale_A8=A8, scores=I, scale_A=A, cand=cand, sel=sel,
                rows=rows_bits, out=out, lse=lse)
