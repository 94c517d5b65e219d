"""Seeded synthetic workloads for the compressed-sparse-attention decode path.

This module draws random numbers, rounds them to bfloat16 and lays them out in
the packed device layout.  It holds none of the scoring, selection, gather or
attention arithmetic, so that both the HIP path and the CPU reference can take
their inputs from it without sharing any of the method.

Layout (row-major, last index fastest):

* ``q_idx``   uint16 (bf16 bits) ``[T, n_ih, ihd]``   indexer queries
* ``w``       float32            ``[T, n_ih]``        indexer head weights
* ``k_idx``   uint16             ``[R, ihd]``         one indexer key per block
* ``comp_kv`` uint16             ``[R, head_dim]``    compressed KV rows
* ``swa``     uint16             ``[S, head_dim]``    sliding-window KV rows
* ``q``       uint16             ``[T, n_heads, head_dim]`` attention queries
* ``pos``     int64 ``[T]``   0-based absolute position of each query token
* ``seq_kv``  int64 ``[T]``   first row of the token's sequence in k_idx/comp_kv
* ``n_comp``  int32 ``[T]``   rows stored for the token's sequence
* ``swa_row0`` int64 ``[T]``  first SWA row of the token
* ``swa_len`` int32 ``[T]``   number of SWA rows of the token

The caches of all sequences are concatenated ("packed"); the per-token arrays
say where each token's sequence starts.  Values are drawn with
``numpy.random.default_rng(seed)`` as float32 standard normals in the fixed
order q_idx, k_idx, w, comp_kv, swa, q; then planted keys.  Every bf16 array
is the round-to-nearest-even image of its float32 draw.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class CSAInputs:
    """One batch of decode (or prefill-chunk) inputs, all host arrays."""

    name: str
    n_ih: int
    ihd: int
    ratio: int
    top_k: int
    window: int
    n_heads: int
    head_dim: int
    scale: float
    q_idx: np.ndarray
    w: np.ndarray
    k_idx: np.ndarray
    comp_kv: np.ndarray
    swa: np.ndarray
    q: np.ndarray
    pos: np.ndarray
    seq_kv: np.ndarray
    n_comp: np.ndarray
    swa_row0: np.ndarray
    swa_len: np.ndarray
    planted: Optional[np.ndarray] = None  # block indices of planted keys (token 0)
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.pos.shape[0])

    def max_visible(self) -> int:
        """Host-side upper bound on visible blocks of any token (for sizing)."""
        return int(np.max(np.minimum(self.pos // self.ratio, self.n_comp)))


def synth(
    seed: int,
    *,
    name: str = "custom",
    pos: Sequence[int],
    seq_of_token: Optional[Sequence[int]] = None,
    n_comp_seq: Sequence[int],
    n_ih: int,
    ihd: int,
    ratio: int,
    top_k: int,
    window: int,
    n_heads: int,
    head_dim: int,
    w_std: float,
    swa_mode: str = "per_token",
    plant: int = 0,
    scale: Optional[float] = None,
) -> CSAInputs:
    """Draw one batch of inputs.

    ``swa_mode="per_token"``: each token owns ``window`` SWA rows at
    ``swa_row0 = t*window``, of which ``min(window, pos+1)`` are filled.
    ``swa_mode="linear"``: the tokens share one linear raw-KV array that covers
    positions ``[min(pos)-window+1, max(pos)]``; token t uses the ``window``
    rows ending at its own position (prefill chunk).
    """
    pos = np.asarray(pos, dtype=np.int64)
    T = int(pos.shape[0])
    if seq_of_token is None:
        seq_of_token = np.zeros(T, dtype=np.int64)
    seq_of_token = np.asarray(seq_of_token, dtype=np.int64)
    n_comp_seq = np.asarray(n_comp_seq, dtype=np.int64)
    starts = np.zeros(len(n_comp_seq), dtype=np.int64)
    if len(n_comp_seq) > 1:
        starts[1:] = np.cumsum(n_comp_seq)[:-1]
    R = int(n_comp_seq.sum())

    if swa_mode == "per_token":
        swa_len = np.minimum(window, pos + 1).astype(np.int32)
        swa_row0 = (np.arange(T, dtype=np.int64) * window)
        S = T * window
    elif swa_mode == "linear":
        base = int(pos.min()) - window + 1
        if base < 0:
            raise ValueError("linear SWA needs pos >= window-1")
        swa_row0 = pos - window + 1 - base
        swa_len = np.full(T, window, dtype=np.int32)
        S = int(pos.max()) - base + 1
    else:
        raise ValueError(swa_mode)

    rng = np.random.default_rng(seed)
    f = np.float32
    q_idx = f32_to_bf16_bits(rng.standard_normal((T, n_ih, ihd), dtype=f))
    k_idx = f32_to_bf16_bits(rng.standard_normal((R, ihd), dtype=f))
    w = (rng.standard_normal((T, n_ih), dtype=f) * f(w_std)).astype(np.float32)
    comp_kv = f32_to_bf16_bits(rng.standard_normal((R, head_dim), dtype=f))
    swa = f32_to_bf16_bits(rng.standard_normal((S, head_dim), dtype=f))
    q = f32_to_bf16_bits(rng.standard_normal((T, n_heads, head_dim), dtype=f))

    planted = None
    if plant:
        # Keys aligned with the token-0 query direction v = sum_h w_h q_h,
        # scaled to the norm sqrt(ihd) of a typical N(0,1) key.
        n_vis0 = int(min(pos[0] // ratio, n_comp_seq[seq_of_token[0]]))
        planted = np.sort(rng.choice(n_vis0, size=plant, replace=False)).astype(np.int64)
        qf = bf16_bits_to_f32(q_idx[0]).astype(np.float64)
        v = (w[0].astype(np.float64)[:, None] * qf).sum(axis=0)
        key = np.sqrt(ihd) * v / np.linalg.norm(v)
        row0 = starts[seq_of_token[0]]
        k_idx[row0 + planted] = f32_to_bf16_bits(key.astype(np.float32))[None, :]

    return CSAInputs(
        name=name, n_ih=n_ih, ihd=ihd, ratio=ratio, top_k=top_k, window=window,
        n_heads=n_heads, head_dim=head_dim,
        scale=float(scale if scale is not None else 1.0 / np.sqrt(head_dim)),
        q_idx=q_idx, w=w, k_idx=k_idx, comp_kv=comp_kv, swa=swa, q=q,
        pos=pos, seq_kv=starts[seq_of_token].astype(np.int64),
        n_comp=n_comp_seq[seq_of_token].astype(np.int32),
        swa_row0=swa_row0.astype(np.int64), swa_len=swa_len.astype(np.int32),
        planted=planted,
    )


def plant_keys(inp: CSAInputs, t: int, blocks: Sequence[int], seed: int,
               jitter: float = 0.05) -> np.ndarray:
    """Overwrite the indexer keys of token t's visible blocks ``blocks`` with
    keys aligned to that token's query direction v = sum_h w_h q_idx[t,h]
    (norm sqrt(ihd), the norm of a typical N(0,1) key) plus independent
    N(0, jitter^2) noise per component, so that the planted blocks stand out
    from the random ones while their own values stay distinct.  Modifies
    ``inp.k_idx`` in place and returns the sorted planted block indices."""
    blocks = np.unique(np.asarray(blocks, dtype=np.int64))
    n_vis = int(min(inp.pos[t] // inp.ratio, inp.n_comp[t]))
    if blocks.size and (blocks.min() < 0 or blocks.max() >= n_vis):
        raise ValueError("planted blocks must be visible to the token")
    qf = bf16_bits_to_f32(inp.q_idx[t]).astype(np.float64)
    v = (inp.w[t].astype(np.float64)[:, None] * qf).sum(axis=0)
    key = np.sqrt(inp.ihd) * v / np.linalg.norm(v)
    rng = np.random.default_rng(seed)
    noise = rng.standard_normal((blocks.size, inp.ihd), dtype=np.float32) * np.float32(jitter)
    rows = (key.astype(np.float32)[None, :] + noise).astype(np.float32)
    inp.k_idx[int(inp.seq_kv[t]) + blocks] = f32_to_bf16_bits(rows)
    return blocks


@dataclass
class HCAInputs:
    """Dense heavily-compressed-attention inputs (ratio 128, no indexer)."""

    name: str
    ratio: int
    n_heads: int
    head_dim: int
    scale: float
    q: np.ndarray        # [T, n_heads, head_dim] bf16 bits
    comp_kv: np.ndarray  # [R, head_dim]
    swa: np.ndarray      # [T*window, head_dim]
    pos: np.ndarray
    seq_kv: np.ndarray
    n_comp: np.ndarray
    swa_row0: np.ndarray
    swa_len: np.ndarray

    @property
    def T(self) -> int:
        return int(self.pos.shape[0])


def synth_hca(seed: int, *, name: str = "hca", pos: Sequence[int], n_comp: int,
              n_heads: int, head_dim: int, window: int, ratio: int = 128) -> HCAInputs:
    """Single-sequence HCA inputs: q, comp_kv, swa drawn in that order."""
    pos = np.asarray(pos, dtype=np.int64)
    T = int(pos.shape[0])
    rng = np.random.default_rng(seed)
    f = np.float32
    q = f32_to_bf16_bits(rng.standard_normal((T, n_heads, head_dim), dtype=f))
    comp_kv = f32_to_bf16_bits(rng.standard_normal((n_comp, head_dim), dtype=f))
    swa = f32_to_bf16_bits(rng.standard_normal((T * window, head_dim), dtype=f))
    return HCAInputs(
        name=name, ratio=ratio, n_heads=n_heads, head_dim=head_dim,
        scale=float(1.0 / np.sqrt(head_dim)), q=q, comp_kv=comp_kv, swa=swa, pos=pos,
        seq_kv=np.zeros(T, dtype=np.int64), n_comp=np.full(T, n_comp, dtype=np.int32),
        swa_row0=np.arange(T, dtype=np.int64) * window,
        swa_len=np.minimum(window, pos + 1).astype(np.int32),
    )


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------

MAIN = dict(n_ih=64, ihd=128, ratio=4, top_k=1024, window=128, n_heads=64,
            head_dim=512, w_std=1.0 / 8.0)


def tiny(seed: int = 0) -> CSAInputs:
    """1 token at position 255, ratio 4 (63 visible blocks), n_ih 8, ihd 32,
    top_k 16, window 16, 8 heads x 64; w ~ N(0, 1/8); scale 1/sqrt(64)."""
    return synth(seed, name="tiny", pos=[255], n_comp_seq=[63], n_ih=8, ihd=32,
                 ratio=4, top_k=16, window=16, n_heads=8, head_dim=64,
                 w_std=float(np.sqrt(1.0 / 8.0)))


def ctx32k(seed: int = 1) -> CSAInputs:
    """Batch-1 decode after a 32,768-token context: 8192 blocks, 16 planted keys."""
    return synth(seed, name="32k", pos=[32768], n_comp_seq=[8192], plant=16, **MAIN)


def ctx1m(seed: int = 2) -> CSAInputs:
    """Batch-1 decode after a 2^20-token context: 262,144 blocks."""
    return synth(seed, name="1m", pos=[1 << 20], n_comp_seq=[(1 << 20) // 4], **MAIN)


def hca1m(seed: int = 2) -> HCAInputs:
    """Dense HCA variant at 2^20 tokens: 8192 blocks of ratio 128 + 128 SWA rows."""
    return synth_hca(seed + 1000, name="hca1m", pos=[1 << 20], n_comp=(1 << 20) // 128,
                     n_heads=64, head_dim=512, window=128)


def batched(seed: int = 3, n_seq: int = 32, lo: int = 16384, hi: int = 131072) -> CSAInputs:
    """32 independent sequences, lengths uniform in [lo, hi]; one query each at
    pos = length, so each sees floor(length/4) blocks."""
    lens = np.random.default_rng((seed, 7)).integers(lo, hi, size=n_seq, endpoint=True)
    return synth(seed, name="batched", pos=lens, seq_of_token=np.arange(n_seq),
                 n_comp_seq=lens // 4, **MAIN)


def prefill(seed: int = 4, T: int = 4096, ctx: int = 65536) -> CSAInputs:
    """A chunk of T consecutive query tokens ending at position ctx-1, one
    sequence of ctx/4 stored blocks, SWA taken from a linear raw-KV array."""
    pos = np.arange(ctx - T, ctx, dtype=np.int64)
    return synth(seed, name="prefill", pos=pos, n_comp_seq=[ctx // 4],
                 swa_mode="linear", **MAIN)


WORKLOADS = {"tiny": tiny, "32k": ctx32k, "1m": ctx1m, "batched": batched,
             "prefill": prefill}


# ---------------------------------------------------------------------------
# Producer side (compressors and cache append) of one decode step.
# ---------------------------------------------------------------------------

@dataclass
class ProducerInputs:
    """One decode step's producer inputs and the per-sequence state before it.

    x [T, H] bf16 bits; w_kv [2*hd, H], w_ik [2*ihd, H] bf16 bits (one output
    channel per row, N(0, 1/H)); seq [T] int32 (distinct); pos [T] int64;
    ring [S, 2*ratio, 2*hd + 2*ihd] float32; swa [S, window, hd] bf16 bits;
    swa_head, swa_len, n_comp [S] int32; seq_kv [S] int64; comp_kv
    [rows, hd] and k_idx [rows, ihd] bf16 bits."""

    H: int
    hd: int
    ihd: int
    ratio: int
    window: int
    x: np.ndarray
    w_kv: np.ndarray
    w_ik: np.ndarray
    seq: np.ndarray
    pos: np.ndarray
    ring: np.ndarray
    swa: np.ndarray
    swa_head: np.ndarray
    swa_len: np.ndarray
    n_comp: np.ndarray
    seq_kv: np.ndarray
    comp_kv: np.ndarray
    k_idx: np.ndarray

    @property
    def T(self) -> int:
        return int(self.pos.shape[0])


def producer(seed: int, *, S: int, T: int, H: int, hd: int, ihd: int, ratio: int, window: int,
             max_pos: int) -> ProducerInputs:
    """Draw T tokens of T distinct sequences (of S) at positions in
    [0, max_pos), with a consistent state: n_comp = floor(pos/ratio) stored
    blocks, a window ring holding min(pos, window) rows with its head at
    pos mod window, and a ring of earlier projections drawn as N(0, 1).
    Draw order: x, w_kv, w_ik, ring, swa, comp_kv, k_idx, then the choices."""
    rng = np.random.default_rng(seed)
    f = np.float32
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=f))
    w_kv = f32_to_bf16_bits((rng.standard_normal((2 * hd, H), dtype=f) / np.sqrt(H)).astype(f))
    w_ik = f32_to_bf16_bits((rng.standard_normal((2 * ihd, H), dtype=f) / np.sqrt(H)).astype(f))
    ring = rng.standard_normal((S, 2 * ratio, 2 * hd + 2 * ihd), dtype=f)
    swa = f32_to_bf16_bits(rng.standard_normal((S, window, hd), dtype=f))
    seq = np.sort(rng.choice(S, size=T, replace=False)).astype(np.int32)
    pos_s = rng.integers(0, max_pos, size=S).astype(np.int64)
    n_comp = (pos_s // ratio).astype(np.int32)
    # The compressed caches are represented by their last two rows per
    # sequence (the producer writes only row seq_kv + n_comp): sequence s's
    # block n_comp lands on row 2s + 1, so seq_kv[s] = 2s + 1 - n_comp (the
    # rows of its earlier blocks are not materialised).
    seq_kv = (2 * np.arange(S, dtype=np.int64) + 1 - n_comp.astype(np.int64))
    rows = 2 * S
    comp_kv = f32_to_bf16_bits(rng.standard_normal((rows, hd), dtype=f))
    k_idx = f32_to_bf16_bits(rng.standard_normal((rows, ihd), dtype=f))
    return ProducerInputs(
        H=H, hd=hd, ihd=ihd, ratio=ratio, window=window, x=x, w_kv=w_kv, w_ik=w_ik, seq=seq,
        pos=pos_s[seq], ring=ring, swa=swa, swa_head=(pos_s % window).astype(np.int32),
        swa_len=np.minimum(pos_s, window).astype(np.int32), n_comp=n_comp, seq_kv=seq_kv,
        comp_kv=comp_kv, k_idx=k_idx)


def producer_1m(seed: int = 5, T: int = 1) -> ProducerInputs:
    """The producer of the 1M-context layer: H 7168, hd 512, ihd 128, ratio 4,
    window 128; T sequences (of 64) near 2^20 tokens."""
    return producer(seed, S=64, T=T, H=7168, hd=512, ihd=128, ratio=4, window=128,
                    max_pos=1 << 20)
