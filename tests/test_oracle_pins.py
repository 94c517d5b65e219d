"""Pins of the CPU oracle against facts fixed outside the oracle itself:
hand-worked examples (tests/golden), closed forms, invariants, brute force on
tiny inputs, and the pages' own executable statement of the scorer run as a
torch fp64 program.  Each group is chosen so that a plausible slip in the
oracle (a dropped ReLU or weight, a sign, a transposed operand, an off-by-one
in visibility, a wrong softmax normaliser) fails at least one test."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (bf16_to_f64, visible_blocks, indexer_scores, select_top_blocks,
                    gather_rows, shared_kv_attention, csa_token, hca_token)
from sparse_long_context_index_amd import inputs as gen


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# bf16 decoding
# --------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x3F00, 0x4049, 0x7F7F],
                    dtype=np.uint16)
    want = [1.0, -1.0, 2.0, 0.0, -0.0, 0.5, 3.140625, 3.3895313892515355e38]
    got = bf16_to_f64(bits)
    assert got.tolist() == want


# --------------------------------------------------------------------------
# Visibility (causality)
# --------------------------------------------------------------------------

def test_visibility_hand_cases(golden_dir):
    g = _load(golden_dir, "visibility_hand.json")
    for pos, ratio, n_comp, want in g["cases"]:
        assert visible_blocks(pos, ratio, n_comp) == want, (pos, ratio, n_comp)


def test_visibility_brute_force():
    """Block b (positions b*r .. b*r+r-1) is visible iff every one of its
    positions precedes the query and it is not the query's own block."""
    for ratio in (1, 2, 4, 5, 128):
        for pos in range(0, 700):
            own = pos // ratio
            vis = [b for b in range(0, 200)
                   if all(p < pos for p in range(b * ratio, b * ratio + ratio)) and b != own]
            want = min(len(vis), 150)
            assert visible_blocks(pos, ratio, 150) == want
            assert own not in range(visible_blocks(pos, ratio, 150))


# --------------------------------------------------------------------------
# Indexer scores
# --------------------------------------------------------------------------

def test_indexer_hand_example(golden_dir):
    g = _load(golden_dir, "indexer_hand.json")
    I, A = indexer_scores(np.array(g["q_idx"], float), np.array(g["w"]), np.array(g["keys"], float))
    assert I.tolist() == g["I"]
    assert A.tolist() == g["A"]
    assert select_top_blocks(I, g["top_k"]).tolist() == g["sel"]


def test_indexer_brute_force_tiny():
    inp = gen.tiny()
    n_vis = visible_blocks(int(inp.pos[0]), inp.ratio, int(inp.n_comp[0]))
    q = bf16_to_f64(inp.q_idx[0]).tolist()
    K = bf16_to_f64(inp.k_idx[:n_vis]).tolist()
    w = inp.w[0].astype(np.float64).tolist()
    want = []
    for s in range(n_vis):
        tot = 0.0
        for h in range(inp.n_ih):
            dot = math.fsum(q[h][d] * K[s][d] for d in range(inp.ihd))
            tot += w[h] * (dot if dot > 0 else 0.0)
        want.append(tot)
    I, _ = indexer_scores(bf16_to_f64(inp.q_idx[0]), inp.w[0], bf16_to_f64(inp.k_idx[:n_vis]))
    np.testing.assert_allclose(I, want, rtol=1e-12, atol=1e-12)


def _rand_case(seed, n=200, n_ih=16, ihd=32):
    r = np.random.default_rng(seed)
    return r.standard_normal((n_ih, ihd)), r.standard_normal(n_ih), r.standard_normal((n, ihd))


def test_indexer_linear_in_w():
    q, w, K = _rand_case(1)
    w2 = np.random.default_rng(2).standard_normal(w.shape)
    a, b = -1.7, 0.3
    I1, _ = indexer_scores(q, w, K)
    I2, _ = indexer_scores(q, w2, K)
    I3, _ = indexer_scores(q, a * w + b * w2, K)
    np.testing.assert_allclose(I3, a * I1 + b * I2, rtol=1e-12, atol=1e-12)


def test_indexer_positive_homogeneity_and_relu():
    q, w, K = _rand_case(3)
    I, _ = indexer_scores(q, w, K)
    np.testing.assert_allclose(indexer_scores(2.5 * q, w, K)[0], 2.5 * I, rtol=1e-12, atol=1e-12)
    # a negative scale is NOT a plain sign flip because of the ReLU
    assert not np.allclose(indexer_scores(-q, w, K)[0], -I)
    # non-negative weights give non-negative scores; every term is ReLU >= 0
    Ip, Ap = indexer_scores(q, np.abs(w), K)
    assert (Ip >= 0).all()
    np.testing.assert_allclose(Ip, Ap, rtol=1e-12)
    assert (indexer_scores(q, w, K)[1] >= np.abs(I) - 1e-12).all()


def test_indexer_one_hot_weight_is_single_head_relu():
    """w = e_h reduces the score to ReLU(K q_h): checked against a torch fp64
    matrix-vector product."""
    q, _, K = _rand_case(4)
    for h in (0, 7, 15):
        w = np.zeros(q.shape[0]); w[h] = 1.0
        want = torch.relu(torch.from_numpy(K) @ torch.from_numpy(q[h])).numpy()
        np.testing.assert_allclose(indexer_scores(q, w, K)[0], want, rtol=1e-12, atol=1e-13)


def test_indexer_matches_per_head_torch_products():
    """Post-probe rewrite, F3: every head scores every key with one shared key
    row, the products pass through ReLU, are weighted by the head's w and
    summed over heads, and the top-k is taken over the sums.  Restated here
    head by head with torch fp64 matrix-vector products and torch.topk, and
    compared with the oracle's scores and top-k set."""
    r = np.random.default_rng(5)
    T, n_ih, ihd, n = 3, 8, 32, 300
    q = r.standard_normal((T, n_ih, ihd)); K = r.standard_normal((n, ihd)); w = r.standard_normal((T, n_ih))
    Kt = torch.from_numpy(K)
    for t in range(T):
        total = torch.zeros(n, dtype=torch.float64)
        for h in range(n_ih):
            logits = torch.mv(Kt, torch.from_numpy(q[t, h]))   # [n]: key s . q_h
            total += float(w[t, h]) * torch.clamp(logits, min=0.0)
        _, idx = torch.topk(total, min(40, n))
        I, _ = indexer_scores(q[t], w[t], K)
        np.testing.assert_allclose(I, total.numpy(), rtol=1e-12, atol=1e-12)
        assert set(select_top_blocks(I, 40).tolist()) == set(idx.tolist())


def test_indexer_per_head_key_algebra_differs():
    """Negative control: the refuted per-head-key reading ('tnd,cnd->tnc' with
    n_ih*ihd-wide keys) must not agree with the oracle on the same data."""
    r = np.random.default_rng(6)
    n_ih, ihd, n = 4, 8, 50
    q = r.standard_normal((n_ih, ihd)); w = r.standard_normal(n_ih)
    wide = r.standard_normal((n, n_ih * ihd))
    refuted = (np.maximum(np.einsum("nd,cnd->cn", q, wide.reshape(n, n_ih, ihd)), 0) * w).sum(1)
    ours, _ = indexer_scores(q, w, wide[:, :ihd])
    assert refuted.shape == ours.shape
    assert not np.allclose(refuted, ours)


# --------------------------------------------------------------------------
# Top-k selection
# --------------------------------------------------------------------------

def test_topk_exhaustive_subsets():
    r = np.random.default_rng(7)
    for trial in range(20):
        I = r.standard_normal(10)
        sel = set(select_top_blocks(I, 3).tolist())
        best = max(itertools.combinations(range(10), 3), key=lambda c: sum(I[list(c)]))
        assert sel == set(best)


def test_topk_selection_property_and_causal_bounds():
    r = np.random.default_rng(8)
    I = r.standard_normal(5000)
    sel = select_top_blocks(I, 1024)
    rest = np.setdiff1d(np.arange(5000), sel)
    assert len(sel) == 1024 and len(set(sel.tolist())) == 1024
    assert I[sel].min() >= I[rest].max()
    assert sel.min() >= 0 and sel.max() < 5000


def test_topk_fewer_blocks_than_k_and_empty():
    I = np.array([0.3, -2.0, 5.0])
    assert sorted(select_top_blocks(I, 16).tolist()) == [0, 1, 2]
    assert select_top_blocks(np.zeros(0), 16).tolist() == []


def test_topk_ties_lowest_index():
    assert select_top_blocks(np.array([1.0, 2.0, 2.0, 2.0, 0.0]), 2).tolist() == [1, 2]
    assert select_top_blocks(np.zeros(10), 4).tolist() == [0, 1, 2, 3]


def test_topk_matches_torch_topk_on_distinct_scores():
    I = np.random.default_rng(9).standard_normal(20000)
    _, idx = torch.from_numpy(I).topk(1024)
    assert set(select_top_blocks(I, 1024).tolist()) == set(idx.tolist())


def test_planted_blocks_are_exact_top16_32k():
    inp = gen.ctx32k()
    res_n = visible_blocks(int(inp.pos[0]), inp.ratio, int(inp.n_comp[0]))
    I, _ = indexer_scores(bf16_to_f64(inp.q_idx[0]), inp.w[0], bf16_to_f64(inp.k_idx[:res_n]))
    top16 = select_top_blocks(I, 16)
    assert set(top16.tolist()) == set(inp.planted.tolist())
    others = np.setdiff1d(np.arange(res_n), inp.planted)
    assert I[inp.planted].min() > I[others].max()


# --------------------------------------------------------------------------
# Gather
# --------------------------------------------------------------------------

def test_gather_order_and_content():
    comp = np.arange(10 * 3).reshape(10, 3)
    swa = 100 + np.arange(2 * 3).reshape(2, 3)
    rows = gather_rows(comp, np.array([7, 2, 2 + 3]), swa)
    assert rows.tolist() == [comp[7].tolist(), comp[2].tolist(), comp[5].tolist(),
                             swa[0].tolist(), swa[1].tolist()]
    assert gather_rows(comp, np.zeros(0, int), swa).tolist() == swa.tolist()


# --------------------------------------------------------------------------
# Shared-KV attention
# --------------------------------------------------------------------------

def test_attention_hand_example(golden_dir):
    g = _load(golden_dir, "attention_hand.json")
    q = np.array([[2 * math.log(3), 0.0], [0.0, 0.0], [0.0, 2 * math.log(7)]])
    rows = np.array(g["rows"], float)
    out, lse = shared_kv_attention(q, rows, g["scale"])
    np.testing.assert_allclose(out, g["out"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(np.exp(lse), g["lse_exp"], rtol=1e-14)
    sink = np.log(np.array(g["sink_ln"]))
    out2, lse2 = shared_kv_attention(q, rows, g["scale"], sink)
    np.testing.assert_allclose(out2, g["out_sink"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(np.exp(lse2), g["lse_sink_exp"], rtol=1e-14)


def test_attention_closed_forms():
    r = np.random.default_rng(10)
    rows = r.standard_normal((37, 16))
    # zero query: uniform weights -> mean of the rows, lse = log n
    out, lse = shared_kv_attention(np.zeros((3, 16)), rows, 0.25)
    np.testing.assert_allclose(out, np.broadcast_to(rows.mean(0), (3, 16)), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(37))
    # one row -> that row; identical rows -> that row
    q = r.standard_normal((4, 16))
    np.testing.assert_allclose(shared_kv_attention(q, rows[:1], 0.3)[0], np.broadcast_to(rows[0], (4, 16)), rtol=1e-12)
    np.testing.assert_allclose(shared_kv_attention(q, np.repeat(rows[:1], 9, 0), 0.3)[0],
                               np.broadcast_to(rows[0], (4, 16)), rtol=1e-12)
    # empty row set
    o, l = shared_kv_attention(q, rows[:0], 0.3)
    assert (o == 0).all() and np.isneginf(l).all()


def test_attention_sink_closed_form():
    r = np.random.default_rng(11)
    rows = r.standard_normal((20, 8)); q = r.standard_normal((5, 8)); sink = r.standard_normal(5)
    o, lse = shared_kv_attention(q, rows, 0.7)
    o2, lse2 = shared_kv_attention(q, rows, 0.7, sink)
    Z = np.exp(lse)
    np.testing.assert_allclose(o2, o * (Z / (Z + np.exp(sink)))[:, None], rtol=1e-12)
    np.testing.assert_allclose(lse2, np.log(Z + np.exp(sink)), rtol=1e-12)


def test_attention_row_permutation_invariant():
    r = np.random.default_rng(12)
    rows = r.standard_normal((50, 32)); q = r.standard_normal((6, 32))
    perm = r.permutation(50)
    a = shared_kv_attention(q, rows, 0.2)
    b = shared_kv_attention(q, rows[perm], 0.2)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13)


def test_attention_matches_torch_sdpa_fp64():
    """Page 3's method: compare against PyTorch SDPA on the same rows (K = V)."""
    r = np.random.default_rng(13)
    rows = r.standard_normal((300, 64)); q = r.standard_normal((8, 64))
    qt = torch.from_numpy(q)[None, :, None, :]          # [B, H, 1, D]
    kv = torch.from_numpy(rows)[None, None].expand(1, 8, 300, 64)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kv, kv, scale=0.125)[0, :, 0]
    np.testing.assert_allclose(shared_kv_attention(q, rows, 0.125)[0], want.numpy(), rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# End to end
# --------------------------------------------------------------------------

def test_csa_equals_hca_when_all_blocks_selected():
    """When n_vis <= top_k the indexer selects every visible block, so CSA
    attends over exactly the dense row set (up to order)."""
    inp = gen.synth(21, pos=[255], n_comp_seq=[63], n_ih=8, ihd=32, ratio=4, top_k=64,
                    window=16, n_heads=8, head_dim=64, w_std=0.35)
    res = csa_token(inp, 0)
    assert len(res["sel"]) == 63
    o, l = hca_token(inp.q[0], inp.comp_kv, 63, inp.swa[:16], inp.scale)
    np.testing.assert_allclose(res["out"], o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res["lse"], l, rtol=1e-13)


def test_csa_causal_perturbation():
    """Keys and rows of blocks at or after the query's own block never matter."""
    inp = gen.tiny()
    a = csa_token(inp, 0)
    inp.k_idx = inp.k_idx.copy(); inp.comp_kv = inp.comp_kv.copy()
    big = np.concatenate([inp.k_idx, gen.f32_to_bf16_bits(np.full((5, inp.ihd), 50.0, np.float32))])
    inp.k_idx = big
    inp.comp_kv = np.concatenate([inp.comp_kv, gen.f32_to_bf16_bits(np.full((5, inp.head_dim), 9.0, np.float32))])
    inp.n_comp = np.array([68], np.int32)   # stored beyond the visible range
    b = csa_token(inp, 0)
    assert b["n_vis"] == 63
    assert a["sel"].tolist() == b["sel"].tolist()
    np.testing.assert_array_equal(a["out"], b["out"])


def test_tiny_end_to_end_shapes():
    inp = gen.tiny()
    r = csa_token(inp, 0)
    assert r["n_vis"] == 63 and len(r["sel"]) == 16 and r["rows"].shape == (32, 64)
    assert r["out"].shape == (8, 64) and np.isfinite(r["lse"]).all()


def _unpacked_token(inp, t):
    """Token t of a packed batch rebuilt as a batch of its own: only its own
    sequence's key and row caches and its own SWA rows, every offset zero."""
    import dataclasses
    row0, n = int(inp.seq_kv[t]), int(inp.n_comp[t])
    s0, sl = int(inp.swa_row0[t]), int(inp.swa_len[t])
    return dataclasses.replace(
        inp, q_idx=inp.q_idx[t:t + 1], w=inp.w[t:t + 1], q=inp.q[t:t + 1],
        k_idx=inp.k_idx[row0:row0 + n].copy(), comp_kv=inp.comp_kv[row0:row0 + n].copy(),
        swa=inp.swa[s0:s0 + sl].copy(), pos=inp.pos[t:t + 1].copy(),
        seq_kv=np.zeros(1, np.int64), n_comp=inp.n_comp[t:t + 1].copy(),
        swa_row0=np.zeros(1, np.int64), swa_len=inp.swa_len[t:t + 1].copy(), planted=None)


def test_csa_token_packed_offsets_match_the_token_alone():
    """Packed batches (1M-context audit, D3/D5: each sequence's compressed rows
    and its sliding window are its own): a token whose key and row caches
    start at seq_kv > 0 and whose SWA rows start at swa_row0 > 0 selects and
    attends exactly as the same token with only its own caches.  The three
    sequences' caches are drawn independently, so an offset slip reads
    another sequence's rows; the negative control shifts seq_kv by one row."""
    inp = gen.synth(31, pos=[201, 333, 250], seq_of_token=[0, 1, 2], n_comp_seq=[50, 83, 62],
                    n_ih=8, ihd=32, ratio=4, top_k=24, window=16, n_heads=8, head_dim=64,
                    w_std=0.35)
    assert inp.seq_kv.tolist() == [0, 50, 133] and inp.swa_row0.tolist() == [0, 16, 32]
    for t in (1, 2):
        packed = csa_token(inp, t)
        alone = csa_token(_unpacked_token(inp, t), 0)
        assert packed["n_vis"] == alone["n_vis"] == min(int(inp.pos[t]) // 4, int(inp.n_comp[t]))
        assert packed["sel"].tolist() == alone["sel"].tolist()
        np.testing.assert_array_equal(packed["rows"], alone["rows"])
        np.testing.assert_array_equal(packed["out"], alone["out"])
        np.testing.assert_array_equal(packed["lse"], alone["lse"])
    shifted = gen.synth(31, pos=[201, 333, 250], seq_of_token=[0, 1, 2], n_comp_seq=[50, 83, 62],
                        n_ih=8, ihd=32, ratio=4, top_k=24, window=16, n_heads=8, head_dim=64,
                        w_std=0.35)
    shifted.seq_kv = shifted.seq_kv + np.array([0, 1, 0])
    bad = csa_token(shifted, 1)
    assert not np.allclose(bad["out"], csa_token(inp, 1)["out"])


def test_hca_token_over_blocks_enumerated_by_causality():
    """Dense HCA (1M-context audit, D4) of a query at position pos attends over
    every stored block that ends before the query's own block begins (PART A,
    suspect 3), then the SWA rows.  The visible set is enumerated block by
    block from that definition, and the softmax is written out per head with
    exp and sums (no max shift at these magnitudes)."""
    r = np.random.default_rng(41)
    H, D, window = 4, 32, 8
    for pos, ratio, n_comp in [(0, 4, 10), (3, 4, 10), (4, 4, 10), (37, 4, 10), (37, 4, 6),
                               (1000, 128, 9), (1151, 128, 9), (1152, 128, 9)]:
        comp = gen.f32_to_bf16_bits(r.standard_normal((n_comp + 3, D), dtype=np.float32))
        swa = gen.f32_to_bf16_bits(r.standard_normal((window, D), dtype=np.float32))
        q = gen.f32_to_bf16_bits(r.standard_normal((H, D), dtype=np.float32))
        own_block_start = (pos // ratio) * ratio
        vis = [b for b in range(n_comp + 3)
               if b < n_comp and (b + 1) * ratio - 1 < own_block_start]
        rows = np.concatenate([bf16_to_f64(comp)[vis], bf16_to_f64(swa)], axis=0)
        qd = bf16_to_f64(q)
        scale = 1.0 / math.sqrt(D)
        expect = np.zeros((H, D))
        for h in range(H):
            e = np.array([math.exp(scale * float(qd[h] @ rows[j])) for j in range(rows.shape[0])])
            expect[h] = (e[:, None] * rows).sum(axis=0) / e.sum()
        o, _ = hca_token(q, comp, visible_blocks(pos, ratio, n_comp), swa, scale)
        assert visible_blocks(pos, ratio, n_comp) == len(vis)
        np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-13)
