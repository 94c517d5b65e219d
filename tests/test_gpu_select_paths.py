"""GPU parity of csa_decode_step on inputs built to drive each path of its
causal top-k (post-probe audit, F3: tk = min(top_k, n_comp) and a top-k over
the indexer scores; PART A, suspect 3: only blocks before the query's own
block are candidates).

The step's select does not look at every score of a long row.  The indexer
keeps, per group of consecutive blocks, a short list of that group's best
blocks and a bound on the rest; the select finds the k-th largest listed key
and then has to handle the groups whose bound reaches it:

* re-scan: a few groups may hold unlisted blocks at or above the threshold;
  their blocks are taken in full and the threshold is found again;
* global: too many blocks to re-scan (or lists too short to hold k keys); the
  select runs over the whole row of scores;
* ties: with w = 0 every score is exactly 0 and the lower block index wins.

Random N(0,1) inputs never reach the first two, so each test plants keys
aligned with the token's indexer query (a few high scores, clustered or
spread) or zeroes the head weights.  Each compares scores, the top-k set (lower
index wins ties), the gathered rows (bit-exact) and the attention output with
the oracle, as the other decode-step tests do.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, indexer_scores, select_top_blocks, visible_blocks
from sparse_long_context_index_amd import inputs as gen
from tests._parity import check_attention, check_step, ref_scores, say

pytestmark = pytest.mark.gpu

ONE_M = 1 << 20


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_index_amd import binding
    binding.load()
    return torch.device("cuda:0")


def run(inp, dev):
    from sparse_long_context_index_amd import binding
    return binding.run_decode_step(inp, dev)


def ctx1m(seed, w_std=None):
    kw = dict(gen.MAIN)
    if w_std is not None:
        kw["w_std"] = w_std
    return gen.synth(seed, name="1m", pos=[ONE_M], n_comp_seq=[ONE_M // 4], **kw)


def test_step_1m_clustered_top_blocks_rescan(dev):
    """The 1024 best blocks are contiguous (70,001 .. 71,024): the two groups
    of 1024 blocks holding them list only a few of theirs, so their bounds reach
    the threshold and they are re-scanned whole (2048 blocks)."""
    say("step 1M: 1024 contiguous planted blocks (group re-scan)")
    inp = ctx1m(21)
    planted = gen.plant_keys(inp, 0, np.arange(70001, 71025), seed=1)
    res = run(inp, dev)
    check_step(inp, res)
    assert res["idx"][0].tolist() == planted.tolist()


def test_step_1m_all_ties_global(dev):
    """w = 0: every score is exactly 0.  All listed keys tie, the first 64
    groups are flagged (65,536 blocks, too many to re-scan), and the select
    runs over the whole row; the lowest 1024 block indices win."""
    say("step 1M: w = 0, all scores tie (global select)")
    inp = ctx1m(22, w_std=0.0)
    res = run(inp, dev)
    check_step(inp, res)
    assert (res["scores"][0] == 0).all()
    assert res["idx"][0].tolist() == list(range(1024))


def test_step_1m_spread_groups_global(dev):
    """24 planted blocks in each of 8 groups spread over the row: each of those
    groups lists 16 and its bound (a planted key) reaches the threshold, and
    8 x 1024 blocks exceed what the select re-scans, so it selects over the
    whole row."""
    say("step 1M: 8 groups x 24 planted blocks (global select)")
    inp = ctx1m(23)
    groups = [3, 40, 77, 114, 151, 188, 225, 255]
    r = np.random.default_rng(3)
    blocks = np.concatenate([g * 1024 + r.choice(1024, 24, replace=False) for g in groups])
    planted = gen.plant_keys(inp, 0, blocks, seed=2)
    res = run(inp, dev)
    check_step(inp, res)
    assert set(planted.tolist()) <= set(res["idx"][0].tolist())


def test_step_1m_threshold_group_partially_listed(dev):
    """The k-th largest block sits inside a planted run that its group lists
    only in part: 1100 contiguous planted blocks over three groups, all three
    re-scanned, and the threshold falls among the planted blocks of one group."""
    say("step 1M: 1100 contiguous planted blocks (threshold inside a re-scanned group)")
    inp = ctx1m(24)
    gen.plant_keys(inp, 0, np.arange(130000, 131100), seed=4, jitter=0.01)
    res = run(inp, dev)
    check_step(inp, res)


def test_step_small_batch_list_paths(dev):
    """Four sequences of 64K..80K tokens: per-wave lists of 32 keys over
    64-block groups (no merging).
      token 0: 1024 contiguous planted blocks (16 groups re-scanned);
      token 1: w = 0, all ties (the first 31 groups re-scanned, lowest indices win);
      token 2: random (no group flagged);
      token 3: 20 whole groups planted, spread over the row (1280 blocks; the
               20 groups are re-scanned)."""
    say("step small batch: clustered / ties / random / spread")
    inp = gen.batched(25, n_seq=4, lo=65536, hi=81920)
    planted0 = gen.plant_keys(inp, 0, np.arange(3000, 4024), seed=5)
    inp.w[1] = 0.0
    r = np.random.default_rng(6)
    n3 = visible_blocks(int(inp.pos[3]), 4, int(inp.n_comp[3]))
    gsel = r.choice(n3 // 64, 20, replace=False)
    planted3 = gen.plant_keys(inp, 3, np.concatenate([g * 64 + np.arange(64) for g in gsel]), seed=7)
    res = run(inp, dev)
    check_step(inp, res)
    assert res["idx"][0].tolist() == planted0.tolist()
    assert res["idx"][1].tolist() == list(range(1024))
    assert set(res["idx"][3].tolist()) <= set(planted3.tolist())


def test_step_long_and_medium_rows(dev):
    """A 1M-context token next to one with 15,000 visible blocks: the shorter
    row's lists (16 keys per 1024-block group, the plan of the long row) hold
    fewer keys than top_k, so its select runs over its whole row while the
    long row uses its lists."""
    say("step T=2: 262,144 and 15,000 visible blocks")
    inp = gen.synth(26, pos=[ONE_M, 4 * 15000 + 1], seq_of_token=[0, 1],
                    n_comp_seq=[ONE_M // 4, 15000], **gen.MAIN)
    res = run(inp, dev)
    check_step(inp, res)


def test_step_keys_out_of_range_select_nothing(dev):
    """seq_kv + n_vis beyond the key buffer: the indexer flags the token and
    scores no block; the step then selects nothing and attends over the SWA
    rows only (the flag is the error word's KEY_RANGE bit)."""
    say("step: keys out of range -> count 0, SWA-only attention")
    inp = gen.synth(27, pos=[401, 399], seq_of_token=[0, 1], n_comp_seq=[100, 100], n_ih=8,
                    ihd=32, ratio=4, top_k=16, window=8, n_heads=8, head_dim=64, w_std=0.3)
    inp.seq_kv[0] = 150  # rows 150..249 of a 200-row buffer
    res = run(inp, dev)
    assert res["err"] & 0x2, f"{res['err']:#x}"
    assert res["count"].tolist() == [0, 16]
    assert (res["idx"][0] == -1).all()
    s0, sl = int(inp.swa_row0[0]), int(inp.swa_len[0])
    check_attention(res["out"][0], inp.q[0], inp.swa[s0:s0 + sl], inp.scale, what="swa-only",
                    lse=res["lse"][0])
    # the other token is unaffected
    res["err"] = 0
    check_step(inp, res, tokens=[1])


def test_step_prefill_many_tokens(dev):
    """The 4096-token prefill chunk: scores and top-k sets of 520 tokens (every
    8th token and the last eight, which covers every token of each indexer
    workgroup slot pattern), attention on a sample."""
    say("step prefill: scores + top-k on 520 tokens, attention on 24")
    inp = gen.prefill()
    from sparse_long_context_index_amd import binding
    res = binding.run_decode_step(inp, dev)
    assert res["err"] == 0
    tokens = sorted(set(range(0, inp.T, 8)) | set(range(inp.T - 8, inp.T)))
    from tests._parity import check_scores, check_topk
    recalls = []
    for t in tokens:
        n, I, A = ref_scores(inp, t)
        check_scores(res["scores"][t, :n], I, A, f"scores t={t}")
        recalls.append(check_topk(res["idx"][t], int(res["count"][t]), I, A, inp.top_k,
                                  f"top-k t={t}"))
    say(f"  mean recall {np.mean(recalls):.5f}")
    check_step(inp, res, tokens=tokens[::22] + [inp.T - 1])
