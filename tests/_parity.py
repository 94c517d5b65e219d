"""Acceptance rules shared by the GPU parity tests.

* scores: |I_gpu - I_ref| <= 1e-3 * max(|I_ref|, A_ref), A = sum_h |w_h| ReLU(.),
  the magnitude the fp32 sum is built from;
* top-k: same count; every block in the symmetric difference of the GPU and
  oracle sets scores within 1e-4 * max(|I_kth|, A_kth) of the k-th score;
* attention (on the GPU's own gathered rows): max |out_gpu - out_ref| <= 2e-2
  and cosine >= 0.9999 per head, bf16 output.
"""
import sys

import numpy as np

from oracle import indexer_scores, select_top_blocks, shared_kv_attention, bf16_to_f64, visible_blocks

SCORE_REL = 1e-3
TIE_REL = 1e-4
ATT_ABS = 2e-2
ATT_COS = 0.9999


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ref_scores(inp, t):
    row0 = int(inp.seq_kv[t])
    n_vis = visible_blocks(int(inp.pos[t]), inp.ratio, int(inp.n_comp[t]))
    I, A = indexer_scores(bf16_to_f64(inp.q_idx[t]), inp.w[t],
                          bf16_to_f64(inp.k_idx[row0:row0 + n_vis]))
    return n_vis, I, A


def check_scores(got, I, A, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == I.shape, (what, got.shape, I.shape)
    if I.size == 0:
        return 0.0
    bound = SCORE_REL * np.maximum(np.abs(I), A) + 1e-30
    err = np.abs(got - I)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, f"{what}: {bad.size} scores out of tolerance, first {bad[:5]} " \
                          f"got {got[bad[:5]]} want {I[bad[:5]]}"
    return float((err / bound).max())


def check_topk(sel, count, I, A, top_k, what=""):
    n = I.shape[0]
    k_eff = min(top_k, n)
    assert count == k_eff, (what, count, k_eff)
    sel = np.asarray(sel[:count], dtype=np.int64)
    assert len(set(sel.tolist())) == k_eff, f"{what}: duplicate indices"
    if k_eff == 0:
        return 1.0
    assert sel.min() >= 0 and sel.max() < n, f"{what}: index outside the visible range"
    assert (np.diff(sel) > 0).all(), f"{what}: indices not in ascending order"
    ref = select_top_blocks(I, top_k)
    kth = ref[-1]
    band = TIE_REL * max(abs(I[kth]), A[kth])
    diff = np.array(sorted(set(sel.tolist()) ^ set(ref.tolist())), dtype=np.int64)
    if diff.size:
        off = np.abs(I[diff] - I[kth])
        assert (off <= band).all(), f"{what}: {diff.size} differing blocks, worst " \
                                    f"{off.max():.3e} from the k-th score (band {band:.3e})"
    return len(set(sel.tolist()) & set(ref.tolist())) / k_eff


def check_attention(out_bf16_as_f32, q_bits, rows_bits, scale, sink=None, what="", lse=None):
    ref, ref_lse = shared_kv_attention(bf16_to_f64(q_bits), bf16_to_f64(rows_bits), scale, sink)
    got = np.asarray(out_bf16_as_f32, dtype=np.float64)
    err = np.abs(got - ref).max() if got.size else 0.0
    assert err <= ATT_ABS, f"{what}: max abs err {err}"
    rn = (ref ** 2).sum(axis=1)
    zero = rn == 0
    # an all-zero reference (empty row set) must give an all-zero output
    assert np.all(got[zero] == 0), f"{what}: expected zero output for an empty row set"
    num = (got * ref).sum(axis=1)
    den = np.sqrt((got ** 2).sum(axis=1) * rn)
    cos = np.where(zero, 1.0, num / np.where(den > 0, den, 1.0))
    assert cos.min() >= ATT_COS, f"{what}: min cos {cos.min()}"
    if lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness"
        if fin.any():
            assert np.abs(lse[fin] - ref_lse[fin]).max() <= 1e-3 * np.maximum(1, np.abs(ref_lse[fin])).max()
    return float(err), float(cos.min())


def check_step(inp, res, tokens=None, sink=None):
    """Scores, top-k, the gathered all_kv rows (bit-exact) and attention of
    the given tokens of one decode-step result against the oracle; returns the
    mean top-k recall."""
    tokens = range(inp.T) if tokens is None else tokens
    assert res["err"] == 0, f"device error {res['err']:#x}"
    recalls = []
    for t in tokens:
        n, I, A = ref_scores(inp, t)
        check_scores(res["scores"][t, :n], I, A, f"scores t={t}")
        cnt = int(res["count"][t])
        recalls.append(check_topk(res["idx"][t], cnt, I, A, inp.top_k, f"top-k t={t}"))
        sel = res["idx"][t, :cnt]
        # gather: bit-exact against the GPU's own selection
        s0, sl = int(inp.swa_row0[t]), int(inp.swa_len[t])
        rows = np.concatenate([inp.comp_kv[int(inp.seq_kv[t]) + sel], inp.swa[s0:s0 + sl]])
        assert int(res["n_kv"][t]) == len(rows)
        assert np.array_equal(res["all_kv"][t, :len(rows)], rows), f"gather t={t}"
        check_attention(res["out"][t], inp.q[t], rows, inp.scale, sink, what=f"attend t={t}",
                        lse=res["lse"][t])
    return float(np.mean(recalls)) if recalls else 1.0
