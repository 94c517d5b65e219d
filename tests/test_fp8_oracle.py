"""Pins of the FP8 (E4M3) part of the oracle (CPU): the decode and the
row quantisation against hand-worked values, torch's float8_e4m3fn type (a
library routine) and their own definitions."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as F
from oracle import indexer_scores

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand.json")


def test_decode_hand_values():
    g = json.load(open(GOLDEN))
    for d in g["decode"]:
        assert F.e4m3_to_f64(np.array([d["code"]], np.uint8))[0] == d["value"], d
    assert np.isnan(F.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_decode_matches_torch_for_every_code():
    c = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_to_f64(c)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))  # -0 is 0x80


def test_round_hand_values_and_row_scale():
    g = json.load(open(GOLDEN))
    for r in g["round"]:
        assert F._round_e4m3(r["x"]) == r["code"], r
    for r in g["row_scale"]:
        assert F.row_scale_exponent(np.array([r["amax"], -r["amax"] / 3])) == r["e"], r


def _edge_rows(rng):
    x = rng.standard_normal((48, 64)) * np.exp2(rng.integers(-30, 30, (48, 1)))
    x[0] = 0.0
    x[1] = -0.0
    x[2, :] = 448.0 * 2.0 ** 5             # amax exactly on a scale boundary
    x[3, 0] = np.nextafter(448.0, 1e9)     # just above it
    x[4] = (np.arange(64) - 32) * 2.0 ** -9 * 0.5   # ties among subnormal steps
    x[5] = 1.0 + (np.arange(64) % 16) / 16.0        # ties between mantissa steps
    x[6, 0] = 1e-300                       # one tiny element
    return x


def test_vectorised_quantiser_equals_scalar_definition():
    x = _edge_rows(np.random.default_rng(1))
    a, sa = F.quantize_rows_e4m3(x)
    b, sb = F.quantize_rows_e4m3_scalar(x)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_quantiser_codes_equal_torch_rne_cast():
    x = _edge_rows(np.random.default_rng(2))
    codes, scale = F.quantize_rows_e4m3(x)
    y = x / scale[:, None]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_scale_is_the_smallest_power_of_two_that_fits():
    x = _edge_rows(np.random.default_rng(3))
    _, scale = F.quantize_rows_e4m3(x)
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    assert (np.log2(scale) == np.round(np.log2(scale))).all()
    assert (amax[nz] / scale[nz] <= 448.0).all()
    assert (amax[nz] / (scale[nz] / 2) > 448.0).all()
    assert (scale[~nz] == 1.0).all()


def test_round_trip_error_within_half_a_step():
    x = np.random.default_rng(4).standard_normal((32, 128))
    codes, scale = F.quantize_rows_e4m3(x)
    back = F.e4m3_to_f64(codes) * scale[:, None]
    y = np.abs(x / scale[:, None])
    # half a mantissa step: 2**-4 relative for normals, 2**-10 absolute (scaled) below 2**-6
    bound = np.where(y >= 2.0 ** -6, y * 2.0 ** -4, 2.0 ** -10) * scale[:, None]
    assert (np.abs(back - x) <= bound * (1 + 1e-12)).all()


def test_fp8_scores_are_the_scores_of_the_dequantised_inputs():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((8, 32)), rng.standard_normal((40, 32))
    w = rng.standard_normal(8) / math.sqrt(8)
    qc, qs = F.quantize_rows_e4m3(q)
    kc, ks = F.quantize_rows_e4m3(k)
    I, A = F.indexer_scores_e4m3(qc, qs, w, kc, ks)
    # by hand: per block, the key scale factors out of every head's ReLU
    qd = F.e4m3_to_f64(qc)
    kd = F.e4m3_to_f64(kc)
    for s in range(40):
        ref = ks[s] * sum(w[h] * qs[h] * max(0.0, float(qd[h] @ kd[s])) for h in range(8))
        assert I[s] == pytest.approx(ref, rel=1e-12, abs=1e-12)
    # and close to the unquantised scores, relative to the condition scale
    I0, A0 = indexer_scores(q, w, k)
    assert (np.abs(I - I0) <= 0.2 * A0 + 1e-9).all()


# ---------------------------------------------------------------------------
# The E4M3 prefilter's selection rule
# ---------------------------------------------------------------------------

def _dominates(S, vals, n):
    """Every member of S comes before every non-member in the order
    (larger value first, then lower index)."""
    rest = [j for j in range(n) if j not in S]
    return all((vals[a], -a) > (vals[b], -b) for a in S for b in rest)


def test_prefilter_matches_brute_force_on_tiny_rows():
    import itertools
    rng = np.random.default_rng(11)
    for trial in range(40):
        n = int(rng.integers(1, 10))
        top_k = int(rng.integers(1, 5))
        C = int(rng.integers(top_k, top_k + 4))
        # few distinct values, so that ties are frequent
        I8 = rng.integers(0, 4, n).astype(np.float64)
        I = rng.integers(0, 4, n).astype(np.float64)
        sel, cand = F.select_prefiltered(I8, I, top_k, C)
        c_eff, k_eff = min(C, n), min(top_k, n)
        want_c = [set(S) for S in itertools.combinations(range(n), c_eff) if _dominates(S, I8, n)]
        assert len(want_c) == 1
        assert set(cand.tolist()) == want_c[0] and (np.diff(cand) > 0).all()
        Sc = sorted(want_c[0])
        want_k = [set(S) for S in itertools.combinations(Sc, k_eff)
                  if all((I[a], -a) > (I[b], -b) for a in S for b in Sc if b not in S)]
        assert len(want_k) == 1 and set(sel.tolist()) == want_k[0], (trial, I8, I, sel)


def test_prefilter_special_cases():
    rng = np.random.default_rng(12)
    I8 = rng.standard_normal(300)
    I = I8 + 0.3 * rng.standard_normal(300)
    # a prefilter that keeps every block is the plain top-k of the bf16 scores
    sel, _ = F.select_prefiltered(I8, I, 20, 300)
    assert list(sel) == list(indexer_top(I, 20))
    # one that keeps exactly top_k blocks is the top-k of the E4M3 scores
    sel, cand = F.select_prefiltered(I8, I, 20, 20)
    assert set(sel.tolist()) == set(indexer_top(I8, 20).tolist()) == set(cand.tolist())
    assert F.prefilter_count(1024) == 1536 and F.prefilter_count(16) == 24
    assert F.prefilter_count(2048) == 3072 and F.prefilter_count(4000) == 4096


def indexer_top(I, k):
    return np.argsort(-I, kind="stable")[:k]


def test_csa_token_e4m3_keeps_planted_blocks_and_full_recall_at_32k():
    from oracle import csa_token
    from sparse_long_context_index_amd import inputs as gen
    inp = gen.ctx32k()
    r8 = F.csa_token_e4m3(inp, 0)
    r = csa_token(inp, 0)
    assert set(inp.planted.tolist()) <= set(r8["sel"].tolist())
    # the candidates hold the whole bf16 top-k here, so the selections agree
    assert set(r8["sel"].tolist()) == set(r["sel"].tolist())
    # while the E4M3 scores alone would miss part of it
    pure8 = set(indexer_top(r8["scores8"], inp.top_k).tolist())
    assert len(pure8 & set(r["sel"].tolist())) < inp.top_k
    # (both in descending bf16 score order, so the gathered rows agree too)
    assert np.array_equal(r8["rows"], r["rows"])
