"""GPU parity: every C-ABI entry point against the CPU oracle on seeded inputs.

Sizes span several tiles with ragged tails, the degenerate cases (no visible
block, fewer blocks than top_k, all scores equal, empty row sets) and the five
named workloads at their full sizes in the launch configuration the benchmark
uses (the 1M-token decode step is compared in full; the 4096-token prefill
chunk on sampled tokens).
"""
import numpy as np
import pytest
import torch

from oracle import (bf16_to_f64, csa_token, hca_token, select_top_blocks,
                    shared_kv_attention, visible_blocks)
from sparse_long_context_index_amd import inputs as gen
from tests._parity import (check_attention, check_scores, check_step, check_topk, ref_scores,
                           say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_index_amd import binding
    binding.load()
    return torch.device("cuda:0")


def B():
    from sparse_long_context_index_amd import binding
    return binding


def _i64(a, dev):
    return torch.as_tensor(np.asarray(a, dtype=np.int64)).to(dev)


def _i32(a, dev):
    return torch.as_tensor(np.asarray(a, dtype=np.int32)).to(dev)


def _bf(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _err(dev):
    return torch.zeros(1, dtype=torch.int32, device=dev)


# ---------------------------------------------------------------------------
# S1 alone
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ihd,n_ih,lens", [
    (32, 8, [63]),
    (64, 16, [1, 31, 33, 500]),
    (128, 64, [4099, 0, 1000]),
    (128, 100, [777, 64]),
    (128, 128, [2050]),
])
def test_index_score(dev, ihd, n_ih, lens):
    say(f"csa_index_score ihd={ihd} n_ih={n_ih} n_vis={lens}")
    T = len(lens)
    inp = gen.synth(100 + ihd + n_ih, pos=[4 * n for n in lens], seq_of_token=np.arange(T),
                    n_comp_seq=[max(n, 1) + 3 for n in lens], n_ih=n_ih, ihd=ihd, ratio=4,
                    top_k=16, window=8, n_heads=8, head_dim=64, w_std=0.3)
    d = B().upload(inp, dev)
    ld = max(max(lens), 1) + 7
    scores = torch.full((T, ld), -7.0, dtype=torch.float32, device=dev)
    err = _err(dev)
    B().csa_index_score(d["q_idx"], d["w"], d["k_idx"], d["pos"], d["seq_kv"], d["n_comp"],
                        n_ih, ihd, 4, scores, ld, err=err)
    s = scores.cpu().numpy()
    assert int(err.item()) == 0
    for t in range(T):
        n, I, A = ref_scores(inp, t)
        assert n == lens[t]
        check_scores(s[t, :n], I, A, f"token {t}")
        assert (s[t, n:] == -7.0).all(), "wrote beyond n_vis"


def test_index_score_flags_out_of_range_keys(dev):
    say("csa_index_score with seq_kv + n_vis beyond k_rows (flag, no access)")
    inp = gen.synth(5, pos=[400], n_comp_seq=[100], n_ih=8, ihd=32, ratio=4, top_k=16,
                    window=8, n_heads=8, head_dim=64, w_std=0.3)
    d = B().upload(inp, dev)
    d["seq_kv"] = _i64([50], dev)  # rows 50..149 of a 100-row buffer
    scores = torch.full((1, 100), 3.0, device=dev)
    err = _err(dev)
    B().csa_index_score(d["q_idx"], d["w"], d["k_idx"], d["pos"], d["seq_kv"], d["n_comp"],
                        8, 32, 4, scores, 100, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 0x2
    assert (scores.cpu().numpy() == 3.0).all()


# ---------------------------------------------------------------------------
# S2 alone: on the same fp32 scores the selection is unique (lower index wins
# ties), so GPU and oracle must agree exactly.
# ---------------------------------------------------------------------------

def _topk_case(dev, scores_rows, top_k, what):
    T = len(scores_rows)
    ld = max(max(len(r) for r in scores_rows), 1)
    S = np.full((T, ld), np.nan, dtype=np.float32)
    for t, r in enumerate(scores_rows):
        S[t, :len(r)] = r
    pos = [4 * len(r) + 3 for r in scores_rows]
    ncomp = [len(r) for r in scores_rows]
    sc = torch.from_numpy(S).to(dev)
    idx = torch.full((T, top_k), 99, dtype=torch.int32, device=dev)
    cnt = torch.full((T,), 99, dtype=torch.int32, device=dev)
    ws = torch.empty(B().csa_topk_workspace_bytes(T, ld, top_k), dtype=torch.uint8, device=dev)
    err = _err(dev)
    say(f"csa_topk {what}: T={T} ld={ld} top_k={top_k}")
    B().csa_topk(sc, ld, _i64(pos, dev), _i32(ncomp, dev), 4, top_k, idx, cnt, ws, err=err)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    assert int(err.item()) == 0
    for t, r in enumerate(scores_rows):
        ref = np.sort(select_top_blocks(np.asarray(r, dtype=np.float64), top_k))
        k = len(ref)
        assert cnt[t] == k, (what, t, cnt[t], k)
        assert idx[t, :k].tolist() == ref.tolist(), (what, t)
        assert (idx[t, k:] == -1).all()
    return idx, cnt


def test_topk_random_ragged(dev):
    r = np.random.default_rng(11)
    rows = [r.standard_normal(n).astype(np.float32) * 5 for n in (5000, 1, 0, 1024, 1025, 70000)]
    _topk_case(dev, rows, 1024, "ragged normal")


def test_topk_ties_and_degenerate(dev):
    r = np.random.default_rng(12)
    coarse = np.round(r.standard_normal(20000) * 2).astype(np.float32)       # heavy ties
    equal = np.zeros(9000, dtype=np.float32)                                   # all tied
    negz = np.where(r.random(3000) < 0.5, -0.0, 0.0).astype(np.float32)       # -0 == +0
    neg = -np.abs(r.standard_normal(3000)).astype(np.float32) - 1.0           # all negative
    _topk_case(dev, [coarse, equal, negz, neg], 512, "ties")
    _topk_case(dev, [coarse[:7], equal[:2048]], 2048, "k >= n and k == n")


def test_topk_many_candidates_global_path(dev):
    # more than 4096 scores share the threshold bin -> candidates stay in the workspace
    r = np.random.default_rng(13)
    x = (1.0 + r.random(300000) * 0.2).astype(np.float32)    # all in one top-11-bit bin
    _topk_case(dev, [x], 1000, "one-bin")


def test_topk_clustered_top_blocks(dev):
    """The 1024 best blocks are contiguous: the groups holding them list only
    their top few keys, so they must be re-scanned in full."""
    r = np.random.default_rng(15)
    x = r.standard_normal(262144).astype(np.float32)
    x[70001:71025] = 10.0 + r.random(1024).astype(np.float32)
    _topk_case(dev, [x], 1024, "clustered")


def test_topk_spread_groups_global_path(dev):
    """Four top scores in each of 256 groups: too many groups to re-scan in
    the LDS pool, so the select falls back to the scores in global memory."""
    r = np.random.default_rng(16)
    x = (r.standard_normal(262144) * 0.1).astype(np.float32)
    for g in range(256):
        x[g * 1024 + np.arange(4) * 7] = 5.0 + r.random(4).astype(np.float32)
    _topk_case(dev, [x], 1024, "spread")


def test_topk_all_equal_long_row(dev):
    _topk_case(dev, [np.full(300000, 0.5, dtype=np.float32)], 1024, "equal-300k")


def test_topk_1m_sized(dev):
    r = np.random.default_rng(14)
    _topk_case(dev, [(r.standard_normal(262144) * 8 + 3).astype(np.float32)], 1024, "262144")


# ---------------------------------------------------------------------------
# S3 alone: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("head_dim", [64, 128, 256, 512])
def test_gather_bitexact(dev, head_dim):
    say(f"csa_gather head_dim={head_dim}")
    r = np.random.default_rng(head_dim)
    T, top_k, window = 3, 40, 16
    comp = r.integers(0, 65536, size=(500, head_dim), dtype=np.uint16)
    swa = r.integers(0, 65536, size=(T * window, head_dim), dtype=np.uint16)
    counts = np.array([40, 0, 17], dtype=np.int32)
    swa_len = np.array([16, 5, 0], dtype=np.int32)
    seq = np.array([0, 100, 300], dtype=np.int64)
    idx = np.full((T, top_k), -1, dtype=np.int32)
    for t in range(T):
        idx[t, :counts[t]] = r.choice(150, size=counts[t], replace=False)
    row0 = np.arange(T, dtype=np.int64) * window
    all_kv = torch.zeros((T, top_k + window, head_dim), dtype=torch.bfloat16, device=dev)
    n_kv = torch.zeros(T, dtype=torch.int32, device=dev)
    err = _err(dev)
    B().csa_gather(_bf(comp, dev), _i64(seq, dev), _i32(idx, dev), _i32(counts, dev), top_k,
                   _bf(swa, dev), _i64(row0, dev), _i32(swa_len, dev), window, head_dim,
                   all_kv, n_kv, err=err)
    got = _bits(all_kv)
    assert int(err.item()) == 0
    assert n_kv.cpu().numpy().tolist() == (counts + swa_len).tolist()
    for t in range(T):
        want = np.concatenate([comp[seq[t] + idx[t, :counts[t]]], swa[row0[t]:row0[t] + swa_len[t]]])
        assert np.array_equal(got[t, :len(want)], want)
        assert (got[t, len(want):] == 0).all()


# ---------------------------------------------------------------------------
# S4 alone
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("head_dim,n_heads,lens,two,sink", [
    (64, 8, [[32, 0]], False, False),
    (128, 16, [[100, 0], [1, 0], [0, 0]], False, True),
    (256, 64, [[300, 20], [64, 64]], True, False),
    (512, 64, [[1152, 0]], False, False),
    (512, 100, [[700, 128], [5, 3]], True, True),
    (512, 64, [[8192, 128]], True, False),
    # one head group and long rows: 141 and 256 splits (the combine's split
    # statistics span several slots a lane, its partials several rounds)
    (128, 16, [[9000, 0]], False, True),
    (64, 16, [[16384, 0]], False, False),
])
def test_mqa_attend(dev, head_dim, n_heads, lens, two, sink):
    say(f"csa_mqa_attend D={head_dim} H={n_heads} lens={lens} two={two} sink={sink}")
    r = np.random.default_rng(head_dim + n_heads)
    T = len(lens)
    a_len = np.array([l[0] for l in lens], dtype=np.int32)
    b_len = np.array([l[1] for l in lens], dtype=np.int32)
    a_row0 = np.concatenate([[0], np.cumsum(a_len)[:-1]]).astype(np.int64) + 3
    b_row0 = np.concatenate([[0], np.cumsum(b_len)[:-1]]).astype(np.int64)
    f = lambda *s: gen.f32_to_bf16_bits(r.standard_normal(s, dtype=np.float32))  # noqa: E731
    kv_a = f(int(a_len.sum()) + 5, head_dim)
    kv_b = f(max(int(b_len.sum()), 1), head_dim)
    q = f(T, n_heads, head_dim)
    sk = (r.standard_normal(n_heads) * 2).astype(np.float32) if sink else None
    max_rows = int((a_len + b_len).max())
    scale = 1.0 / np.sqrt(head_dim)
    out = torch.zeros((T, n_heads, head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((T, n_heads), dtype=torch.float32, device=dev)
    ws = torch.empty(max(B().csa_attend_workspace_bytes(T, n_heads, head_dim, max_rows), 1),
                     dtype=torch.uint8, device=dev)
    err = _err(dev)
    B().csa_mqa_attend(_bf(q, dev), n_heads, head_dim, scale, _bf(kv_a, dev), _i64(a_row0, dev),
                       _i32(a_len, dev), max_rows, out,
                       kv_b=_bf(kv_b, dev) if two else None, b_row0=_i64(b_row0, dev) if two else None,
                       b_len=_i32(b_len, dev) if two else None,
                       sink=torch.from_numpy(sk).to(dev) if sink else None, lse=lse, ws=ws, err=err)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    assert int(err.item()) == 0
    for t in range(T):
        rows = kv_a[a_row0[t]:a_row0[t] + a_len[t]]
        if two:
            rows = np.concatenate([rows, kv_b[b_row0[t]:b_row0[t] + b_len[t]]])
        check_attention(o[t], q[t], rows, scale, sk, what=f"token {t}", lse=l[t])


# ---------------------------------------------------------------------------
# S5: whole decode step
# ---------------------------------------------------------------------------

def test_decode_step_tiny(dev):
    say("csa_decode_step tiny (pos 255, 63 blocks, top_k 16)")
    inp = gen.tiny()
    res = B().run_decode_step(inp, dev)
    check_step(inp, res)
    ref = csa_token(inp, 0)
    assert sorted(res["idx"][0, :16].tolist()) == sorted(ref["sel"].tolist())


def test_decode_step_ragged_batch(dev):
    say("csa_decode_step ragged batch")
    lens = [0, 3, 1000, 4097, 77]
    inp = gen.synth(31, pos=[4 * n + 2 for n in lens], seq_of_token=np.arange(5),
                    n_comp_seq=[n + 1 for n in lens], n_ih=64, ihd=128, ratio=4, top_k=128,
                    window=32, n_heads=16, head_dim=128, w_std=0.125)
    res = B().run_decode_step(inp, dev)
    check_step(inp, res)
    assert res["count"].tolist() == [0, 3, 128, 128, 77]


def test_decode_step_sink(dev):
    say("csa_decode_step with attention sink")
    inp = gen.synth(32, pos=[999], n_comp_seq=[300], n_ih=8, ihd=64, ratio=4, top_k=64,
                    window=16, n_heads=8, head_dim=256, w_std=0.35)
    sink = np.linspace(-2, 3, 8).astype(np.float32)
    res = B().run_decode_step(inp, dev, sink=torch.from_numpy(sink).to(dev))
    check_step(inp, res, sink=sink)


def test_decode_step_32k_planted(dev):
    say("csa_decode_step 32K context, 16 planted blocks")
    inp = gen.ctx32k()
    res = B().run_decode_step(inp, dev)
    check_step(inp, res)
    assert set(inp.planted.tolist()) <= set(res["idx"][0, :1024].tolist())


def test_decode_step_1m(dev):
    say("csa_decode_step 1M context (262,144 blocks, top_k 1024, 64x512 attention)")
    inp = gen.ctx1m()
    res = B().run_decode_step(inp, dev)
    recall = check_step(inp, res)
    say(f"  recall vs fp64 oracle: {recall:.5f}")
    assert recall >= 0.997


def test_decode_step_1m_deterministic(dev):
    say("csa_decode_step 1M twice: bitwise equal")
    inp = gen.ctx1m()
    a = B().run_decode_step(inp, dev)
    b = B().run_decode_step(inp, dev)
    for k in ("scores", "idx", "count", "all_kv", "out", "lse"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("e4m3", [False, True])
def test_decode_step_stages_equal_whole_step(dev, e4m3):
    say(f"csa_decode_step_stage INDEX then REST == csa_decode_step (1M, e4m3={e4m3})")
    inp = gen.ctx1m()
    b = B()
    d = b.upload(inp, dev)
    if e4m3:
        d = b.quantize_indexer_e4m3(d)
    res = []
    for staged in (False, True):
        outs = b.alloc_step_outputs(inp, dev)
        a = b.step_args(inp, d, outs, e4m3=e4m3)
        ws = b.step_workspace(a, dev)
        if staged:
            b.csa_decode_step_stage(a, b.CSA_STAGE_INDEX, ws)
            b.csa_decode_step_stage(a, b.CSA_STAGE_REST, ws)
        else:
            b.csa_decode_step(a, ws)
        torch.cuda.synchronize()
        res.append({k: v.cpu() for k, v in outs.items()})
    for k in res[0]:
        x, y = res[0][k], res[1][k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), k
    assert int(res[0]["err"][0]) == 0


def test_decode_step_batched(dev):
    say("csa_decode_step batched: 32 sequences of 16K..128K tokens")
    inp = gen.batched()
    res = B().run_decode_step(inp, dev)
    check_step(inp, res)


@pytest.mark.parametrize("n_seq", [4, 8])
def test_decode_step_small_batch_multitile(dev, n_seq):
    """Small batches of long rows take the fused select-and-attend kernel with
    several 64-row tiles per split (1152 rows over 64 heads: 2 tiles per split
    at 4 tokens, 3 at 8), so the later tiles read their block indices from the
    workgroup's window of the selection."""
    say(f"csa_decode_step small batch: {n_seq} sequences of 64K..80K tokens")
    inp = gen.batched(5, n_seq=n_seq, lo=65536, hi=81920)
    res = B().run_decode_step(inp, dev)
    check_step(inp, res)


def test_decode_step_prefill_sampled(dev):
    say("csa_decode_step prefill chunk: 4096 tokens at 61,440..65,535 (sampled check)")
    inp = gen.prefill()
    res = B().run_decode_step(inp, dev)
    check_step(inp, res, tokens=[0, 1, 2047, 3000, 4094, 4095])
    # every token: count and causality
    nv = np.minimum(inp.pos // 4, inp.n_comp)
    assert (res["count"] == np.minimum(1024, nv)).all()
    assert (res["idx"].max(axis=1) < nv).all()


def test_decode_step_hca_1m(dev):
    say("csa_decode_step HCA mode at 1M (8192 blocks + 128 SWA rows)")
    h = gen.hca1m()
    d = {"q": _bf(h.q, dev), "comp_kv": _bf(h.comp_kv, dev), "swa": _bf(h.swa, dev),
         "pos": _i64(h.pos, dev), "seq_kv": _i64(h.seq_kv, dev), "n_comp": _i32(h.n_comp, dev),
         "swa_row0": _i64(h.swa_row0, dev), "swa_len": _i32(h.swa_len, dev)}
    out = torch.zeros((h.T, h.n_heads, h.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((h.T, h.n_heads), dtype=torch.float32, device=dev)
    err = _err(dev)
    a = B().StepArgs()
    a.mode, a.T, a.ratio, a.window, a.n_heads, a.head_dim = 1, h.T, 128, 128, h.n_heads, h.head_dim
    a.max_vis, a.scale = 8192, h.scale
    for k, v in d.items():
        setattr(a, k, v.data_ptr())
    a.comp_rows, a.swa_rows = h.comp_kv.shape[0], h.swa.shape[0]
    a.out, a.lse, a.err = out.data_ptr(), lse.data_ptr(), err.data_ptr()
    ws = B().step_workspace(a, dev)
    B().csa_decode_step(a, ws)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    n_vis = visible_blocks(int(h.pos[0]), 128, int(h.n_comp[0]))
    rows = np.concatenate([h.comp_kv[:n_vis], h.swa[:128]])
    check_attention(out.float().cpu().numpy()[0], h.q[0], rows, h.scale, what="hca",
                    lse=lse.cpu().numpy()[0])


def test_csa_equals_hca_when_all_selected(dev):
    """n_vis <= top_k: the CSA step (all blocks selected) and the HCA step over
    the same rows give the same attention output (up to rounding order)."""
    say("CSA vs HCA with n_vis <= top_k")
    inp = gen.synth(40, pos=[1000], n_comp_seq=[250], n_ih=16, ihd=64, ratio=4, top_k=256,
                    window=32, n_heads=16, head_dim=128, w_std=0.25)
    res = B().run_decode_step(inp, dev)
    assert res["count"][0] == 250
    d = B().upload(inp, dev)
    outs = {"out": torch.zeros((1, 16, 128), dtype=torch.bfloat16, device=dev),
            "err": _err(dev)}
    a = B().step_args(inp, d, outs, mode=B().CSA_MODE_HCA, max_vis=250)
    ws = B().step_workspace(a, dev)
    B().csa_decode_step(a, ws)
    hca = outs["out"].float().cpu().numpy()[0]
    ref, _ = hca_token(inp.q[0], inp.comp_kv, 250, inp.swa[:32], inp.scale)
    assert np.abs(hca - ref).max() <= 2e-2
    assert np.abs(hca - res["out"][0]).max() <= 2e-2
