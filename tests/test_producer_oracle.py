"""Pins of the producer oracle (CPU): the compressors' softmax pooling, the
overlapped block windows, the bf16 rounding and the decode-time cache append,
against closed forms, library routines (torch), brute force and the
whole-sequence definition."""
import math

import numpy as np
import torch

from oracle import producer_oracle as P
from sparse_long_context_index_amd import inputs as gen


def test_pool_closed_forms():
    r = np.random.default_rng(1)
    c = r.standard_normal((8, 5))
    # equal scores: the plain mean of the tokens
    np.testing.assert_allclose(P.pool(c, np.full((8, 5), 0.7)), c.mean(axis=0), rtol=1e-14)
    # one token far above the rest in every channel: that token's values
    z = np.zeros((8, 5)); z[3] = 800.0
    np.testing.assert_allclose(P.pool(c, z), c[3], rtol=1e-14)
    # one token: itself
    np.testing.assert_allclose(P.pool(c[:1], r.standard_normal((1, 5))), c[0], rtol=1e-14)
    # shifting a channel's scores changes nothing
    z = r.standard_normal((8, 5))
    np.testing.assert_allclose(P.pool(c, z + np.arange(5) * 13.0), P.pool(c, z), rtol=1e-12)


def test_pool_matches_torch_softmax_and_brute_force():
    r = np.random.default_rng(2)
    c = r.standard_normal((6, 4)); z = 3 * r.standard_normal((6, 4))
    want = (torch.softmax(torch.from_numpy(z), dim=0) * torch.from_numpy(c)).sum(0).numpy()
    np.testing.assert_allclose(P.pool(c, z), want, rtol=1e-13)
    for ch in range(4):
        ws = [math.exp(z[j, ch]) for j in range(6)]
        brute = sum(w * c[j, ch] for j, w in enumerate(ws)) / sum(ws)
        assert abs(P.pool(c, z)[ch] - brute) <= 1e-13 * max(1.0, abs(brute))


def test_block_windows():
    assert list(P.block_tokens(0, 4)) == [0, 1, 2, 3]
    assert list(P.block_tokens(1, 4)) == list(range(0, 8))
    assert list(P.block_tokens(5, 4)) == list(range(16, 24))
    assert list(P.block_tokens(5, 4, overlap=False)) == list(range(20, 24))
    # a block's window ends with its own last token: complete once it is seen
    for i in range(6):
        assert P.block_tokens(i, 4)[-1] == 4 * i + 3


def test_bf16_rounding_matches_torch_and_ties():
    r = np.random.default_rng(3)
    # fp32-representable values, for which torch's conversion is one rounding
    # (on other fp64 values it rounds twice, through fp32)
    v = (r.standard_normal(20000) * np.exp(r.uniform(-20, 20, 20000))).astype(np.float32)
    v = v.astype(np.float64)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(P.f64_to_bf16_bits(v), want)
    # exact midpoints between bf16 neighbours go to the even one
    assert P.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80      # 1.0 (even)
    assert P.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82  # up to even
    assert P.f64_to_bf16_bits(np.array([-(1.0 + 2.0 ** -8)]))[0] == 0xBF80
    # just above a midpoint goes up
    assert P.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 0x3F81


def _run_sequence(n_tok, ratio, window, hd, ihd, H, seed):
    r = np.random.default_rng(seed)
    xb = gen.f32_to_bf16_bits(r.standard_normal((n_tok, H)).astype(np.float32))
    wk = gen.f32_to_bf16_bits((r.standard_normal((2 * hd, H)) / np.sqrt(H)).astype(np.float32))
    wi = gen.f32_to_bf16_bits((r.standard_normal((2 * ihd, H)) / np.sqrt(H)).astype(np.float32))
    n_blocks = n_tok // ratio
    st = P.ProducerState(ring=np.zeros((1, 2 * ratio, 2 * hd + 2 * ihd)),
                         swa=np.zeros((1, window, hd), np.uint16), swa_head=[0], swa_len=[0],
                         comp_kv=np.zeros((n_blocks + 2, hd), np.uint16),
                         k_idx=np.zeros((n_blocks + 2, ihd), np.uint16), seq_kv=[1], n_comp=[0])
    for p in range(n_tok):
        P.append_step(st, xb[p:p + 1], [0], [p], wk, wi, hd, ihd, ratio, window)
    return st, xb, wk, wi


def test_incremental_append_equals_whole_sequence_definition():
    hd, ihd, H, ratio, window, n_tok = 6, 4, 32, 4, 8, 23
    st, xb, wk, wi = _run_sequence(n_tok, ratio, window, hd, ihd, H, seed=4)
    from oracle import bf16_to_f64
    x = bf16_to_f64(xb)
    yk, yi = P.project(x, bf16_to_f64(wk)), P.project(x, bf16_to_f64(wi))
    n_blocks = n_tok // ratio
    assert st.n_comp[0] == n_blocks
    want_kv = P.compress_sequence(yk, hd, ratio)
    want_ik = P.compress_sequence(yi, ihd, ratio)
    assert np.array_equal(st.comp_kv[1:1 + n_blocks], P.f64_to_bf16_bits(want_kv))
    assert np.array_equal(st.k_idx[1:1 + n_blocks], P.f64_to_bf16_bits(want_ik))
    assert (st.comp_kv[0] == 0).all() and (st.comp_kv[1 + n_blocks:] == 0).all()
    # the window ring holds the last `window` tokens' value halves, the head
    # pointing at the oldest
    assert st.swa_len[0] == window and st.swa_head[0] == n_tok % window
    for k in range(window):
        tok = n_tok - window + k
        slot = (st.swa_head[0] + k) % window
        assert np.array_equal(st.swa[0, slot], P.f64_to_bf16_bits(yk[tok, :hd]))


def test_projection_is_a_plain_matrix_product():
    r = np.random.default_rng(5)
    x = r.standard_normal((3, 40)); w = r.standard_normal((7, 40))
    want = (torch.from_numpy(x) @ torch.from_numpy(w).T).numpy()
    np.testing.assert_allclose(P.project(x, w), want, rtol=1e-13)
    # a one-hot hidden state picks one column of the weights
    e = np.zeros((1, 40)); e[0, 11] = 1.0
    np.testing.assert_array_equal(P.project(e, w)[0], w[:, 11])
