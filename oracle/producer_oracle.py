"""CPU reference for the producer side of the CSA caches: the compressors and
the cache append of one decode step (test infrastructure only, like the rest
of ``oracle/``: never imported by the library or its binding).

What the pages fix:

* [P2] "ARCHITECTURE & MEMORY AUDIT -- 1M-context viability", D1/D2: a CSA
  layer has two compressors of the same form, ``Compressor(ratio, width, H)``:
  the main one (width hd = 512) and the indexer-key one (width ihd = 128),
  each projecting the H-wide hidden state to 2 x width per token, the
  compressed row being width wide;
* the same page, its closing assessment: CSA compresses overlapped windows of
  2m tokens with softmax weights (m = ratio), HCA non-overlapped windows;
* D5: the sliding window is a ring of ``window`` rows whose head advances by
  one per token, modulo the window, evicting the oldest row once full.

Readings where the pages are silent (stated once more in the design notes):

* the 2 x width projection is a value half c and a score half z; a
  compressed row is, channel by channel, the softmax over the window's tokens
  of z applied as weights to c;
* block i of a CSA layer covers tokens [(i-1)m, (i+1)m) (its own m tokens and
  the previous block's), clipped at 0; it is complete -- and appended as row i
  -- once token (i+1)m - 1 has been seen;
* the token's own sliding-window row is its value half c of the main
  compressor, in bf16;
* the projections run on bf16 hidden states and bf16 weights stored one output
  channel per row ([2 x width, H]); the caches hold bf16.
"""
from __future__ import annotations

import numpy as np

from .csa_oracle import bf16_to_f64


def project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[t, n] = sum_k x[t, k] w[n, k]: the compressor's per-token projection
    (fp64 on the given values)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def pool(c: np.ndarray, z: np.ndarray) -> np.ndarray:
    """One compressed row from a window's tokens: per channel, the softmax
    over the tokens of z weighting c.  c, z: [tokens, width]."""
    c = np.asarray(c, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=0, keepdims=True))
    return (e * c).sum(axis=0) / e.sum(axis=0)


def block_tokens(i: int, ratio: int, overlap: bool = True) -> range:
    """Tokens of compressed block i: [(i-1)m, (i+1)m) clipped at 0 when the
    windows overlap (CSA), [im, (i+1)m) otherwise (HCA)."""
    lo = (i - 1) * ratio if overlap else i * ratio
    return range(max(lo, 0), (i + 1) * ratio)


def compress_sequence(y: np.ndarray, width: int, ratio: int, overlap: bool = True) -> np.ndarray:
    """Every complete block of a sequence from the projections y [n_tok,
    2 x width] of all its tokens: row i pools block_tokens(i)."""
    n_blocks = y.shape[0] // ratio
    out = np.zeros((n_blocks, width))
    for i in range(n_blocks):
        toks = list(block_tokens(i, ratio, overlap))
        out[i] = pool(y[toks, :width], y[toks, width:])
    return out


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 bits, nearest with ties to even, decided
    on the fp64 value itself: the bf16 quantum at v's binade is 2**(E-7)
    (2**-133 below the normal range), and rint of v / quantum rounds half to
    even.  The rounded value is exact in fp32, whose upper 16 bits are then
    the bf16 bits.  (Finite values inside the bf16 range.)"""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(np.where(a > 0, a, 1.0))      # a = f * 2**e, 0.5 <= f < 1
    q = np.exp2(np.maximum(e - 1 - 7, -133).astype(np.float64))
    r = np.rint(a / q) * q
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.signbit(v), bits | 0x8000, bits).astype(np.uint16)


class ProducerState:
    """The per-sequence state the decode-time producer keeps and advances:
    a ring of the last 2m tokens' projections of both compressors (fp64 here,
    [S, 2m, 2hd + 2ihd]), the sliding window ring [S, window, hd] (bf16 bits)
    with its head and length, the compressed caches (bf16 bits, packed at
    seq_kv[s]) and n_comp."""

    def __init__(self, ring, swa, swa_head, swa_len, comp_kv, k_idx, seq_kv, n_comp):
        self.ring = np.array(ring, dtype=np.float64)
        self.swa = np.array(swa, dtype=np.uint16)
        self.swa_head = np.array(swa_head, dtype=np.int64)
        self.swa_len = np.array(swa_len, dtype=np.int64)
        self.comp_kv = np.array(comp_kv, dtype=np.uint16)
        self.k_idx = np.array(k_idx, dtype=np.uint16)
        self.seq_kv = np.array(seq_kv, dtype=np.int64)
        self.n_comp = np.array(n_comp, dtype=np.int64)


def append_step(st: ProducerState, x_bits, seq, pos, w_kv_bits, w_ik_bits, hd: int, ihd: int,
                ratio: int, window: int) -> dict:
    """One decode step of the producer for tokens of distinct sequences:

    1. both compressors project the token's hidden state;
    2. the projections go to ring slot pos % 2m of the token's sequence;
    3. the token's value half c (bf16) is appended to its sliding window at the
       head, which then advances modulo the window;
    4. if the token completes block i = (pos+1)/m - 1, both compressors pool
       block_tokens(i) from the ring into row seq_kv + i of comp_kv and k_idx,
       and n_comp becomes i + 1.

    Returns the fp64 projections and pooled rows (before bf16 rounding), for
    tolerance checks.  Mutates st."""
    x = bf16_to_f64(x_bits)
    yk = project(x, bf16_to_f64(w_kv_bits))
    yi = project(x, bf16_to_f64(w_ik_bits))
    y = np.concatenate([yk, yi], axis=1)
    R = 2 * ratio
    pooled = {}
    for t in range(x.shape[0]):
        s, p = int(seq[t]), int(pos[t])
        st.ring[s, p % R] = y[t]
        h = int(st.swa_head[s])
        st.swa[s, h] = f64_to_bf16_bits(yk[t, :hd])
        st.swa_head[s] = (h + 1) % window
        st.swa_len[s] = min(int(st.swa_len[s]) + 1, window)
        if (p + 1) % ratio == 0:
            i = (p + 1) // ratio - 1
            toks = list(block_tokens(i, ratio, True))
            rows = st.ring[s, [j % R for j in toks]]
            e_kv = pool(rows[:, :hd], rows[:, hd:2 * hd])
            e_ik = pool(rows[:, 2 * hd:2 * hd + ihd], rows[:, 2 * hd + ihd:])
            r = int(st.seq_kv[s]) + i
            st.comp_kv[r] = f64_to_bf16_bits(e_kv)
            st.k_idx[r] = f64_to_bf16_bits(e_ik)
            st.n_comp[s] = i + 1
            pooled[t] = (e_kv, e_ik, rows)
    return {"y": y, "pooled": pooled}
