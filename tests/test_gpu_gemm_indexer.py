"""The indexer of many tokens of one sequence as one GEMM (one_sequence = 1:
a prefill chunk's key tiles staged once for eight tokens), against the oracle
and against the per-token indexer on the same inputs.  The scores are the
same operations in the same order, so the two must agree bit for bit."""
import numpy as np
import pytest
import torch

from sparse_long_context_index_amd import inputs as gen
from tests._parity import check_scores, check_step, check_topk, ref_scores, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_index_amd import binding
    binding.load()
    return torch.device("cuda:0")


def _run(inp, dev, one_sequence, all_kv=False):
    from sparse_long_context_index_amd import binding
    return binding.run_decode_step(inp, dev, all_kv=all_kv, one_sequence=one_sequence)


def _same_visible_scores(a, b, inp, tokens):
    for t in tokens:
        n = min(int(inp.pos[t]) // inp.ratio, int(inp.n_comp[t]))
        np.testing.assert_array_equal(a["scores"][t, :n], b["scores"][t, :n], err_msg=f"t={t}")


def test_prefill_one_sequence_matches_per_token_indexer_and_oracle(dev):
    say("prefill chunk, 4096 tokens: GEMM indexer (one_sequence) vs per-token indexer vs oracle")
    inp = gen.prefill()
    gemm = _run(inp, dev, True, all_kv=True)
    tok = _run(inp, dev, False)
    assert gemm["err"] == 0 and tok["err"] == 0
    _same_visible_scores(gemm, tok, inp, range(inp.T))
    np.testing.assert_array_equal(gemm["count"], tok["count"])
    np.testing.assert_array_equal(gemm["idx"], tok["idx"])
    np.testing.assert_array_equal(gemm["out"], tok["out"])
    # the oracle on tokens spread over every position of a workgroup's eight
    # and over the chunk
    tokens = sorted(set(range(0, inp.T, 61)) | set(range(8 * 300, 8 * 300 + 8)) | {inp.T - 1})
    for t in tokens:
        n, I, A = ref_scores(inp, t)
        check_scores(gemm["scores"][t, :n], I, A, f"scores t={t}")
        check_topk(gemm["idx"][t], int(gemm["count"][t]), I, A, inp.top_k, f"top-k t={t}")
    check_step(inp, gemm, tokens=tokens[::9])


def _two_sequences(split, seed, n_ih=64, ihd=128, T=640, base=(4096, 3000), top_k=256):
    # tokens [0, split) of sequence 0, [split, T) of sequence 1, consecutive
    # positions in each from base[0] and base[1]
    pos = np.concatenate([base[0] + np.arange(split), base[1] + np.arange(T - split)])
    return gen.synth(seed, pos=pos, seq_of_token=[0] * split + [1] * (T - split),
                     n_comp_seq=[base[0] // 4 + split // 4 + 1, base[1] // 4 + (T - split) // 4 + 1],
                     n_ih=n_ih, ihd=ihd, ratio=4, top_k=top_k, window=64, n_heads=16,
                     head_dim=128, w_std=1.0 / np.sqrt(n_ih), swa_mode="per_token")


def test_one_sequence_broken_inside_a_workgroup(dev):
    """One_sequence promised but broken: a workgroup of eight tokens takes the
    key rows of its first token, so the tokens of the other sequence in that
    workgroup (604..607 here: the workgroup is tokens 600..607) score no block
    and the error word carries BAD_META; every other token is scored as
    without the promise (the workgroups wholly in one sequence are exact)."""
    say("one_sequence broken: 640 tokens, sequences split at token 604")
    inp = _two_sequences(604, 71)
    gemm = _run(inp, dev, True)
    tok = _run(inp, dev, False)
    assert tok["err"] == 0
    assert gemm["err"] & 0x4  # CSA_DERR_BAD_META
    bad = list(range(604, 608))
    assert (gemm["count"][bad] == 0).all()
    good = [t for t in range(inp.T) if t not in bad]
    _same_visible_scores(gemm, tok, inp, good)
    np.testing.assert_array_equal(gemm["count"][good], tok["count"][good])
    np.testing.assert_array_equal(gemm["idx"][good], tok["idx"][good])


def test_one_sequence_with_short_rows_takes_the_batch_indexer(dev):
    """64 tokens whose rows are short take the batch indexer even with the
    promise: a token of another sequence is then scored on its own rows, and
    the select does not drop it (no BAD_META; every output as without the
    promise)."""
    say("one_sequence with short rows: 64 tokens, batch indexer, split at token 61")
    inp = _two_sequences(61, 74, T=64, top_k=128)
    a = _run(inp, dev, True)
    b = _run(inp, dev, False)
    assert a["err"] == 0 and b["err"] == 0
    _same_visible_scores(a, b, inp, range(inp.T))
    np.testing.assert_array_equal(a["count"], b["count"])
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["out"], b["out"])
    assert (a["count"][61:] > 0).all()


def test_gemm_indexer_four_tile_groups(dev):
    """64 tokens of one sequence over about 75,000 blocks: batches of up to
    512 tokens plan four tiles a wave, so the GEMM kernel's groups are four
    tiles (two steps) and its lists six keys (top_k 512: per-wave lists,
    not merged).  Bit-equal to the per-token indexer; scores and top-k of
    three tokens against the oracle."""
    say("GEMM indexer, four-tile groups: 64 tokens, ~75K blocks, top_k 512")
    inp = _two_sequences(64, 75, T=64, top_k=512, base=(300000, 0))
    gemm = _run(inp, dev, True)
    tok = _run(inp, dev, False)
    assert gemm["err"] == 0 and tok["err"] == 0
    _same_visible_scores(gemm, tok, inp, range(inp.T))
    np.testing.assert_array_equal(gemm["count"], tok["count"])
    np.testing.assert_array_equal(gemm["idx"], tok["idx"])
    np.testing.assert_array_equal(gemm["out"], tok["out"])
    for t in (0, 37, 63):
        n, I, A = ref_scores(inp, t)
        check_scores(gemm["scores"][t, :n], I, A, f"scores t={t}")
        check_topk(gemm["idx"][t], int(gemm["count"][t]), I, A, inp.top_k, f"top-k t={t}")


@pytest.mark.parametrize("n_ih,ihd", [(32, 64), (20, 128)])
def test_gemm_indexer_other_shapes(dev, n_ih, ihd):
    """The GEMM indexer's other instantiations (32 heads or fewer; 64-wide
    keys) on one sequence of rows over 12,288 blocks (so that the select
    works from the candidate lists the GEMM kernel builds): against the
    oracle."""
    say(f"GEMM indexer n_ih={n_ih} ihd={ihd}: 640 tokens of one sequence, ~13,100 blocks")
    inp = _two_sequences(640, 72 + n_ih, n_ih=n_ih, ihd=ihd, base=(52000, 0))
    assert inp.max_visible() > 12288
    gemm = _run(inp, dev, True)
    assert gemm["err"] == 0
    for t in list(range(0, inp.T, 37)) + [inp.T - 1]:
        n, I, A = ref_scores(inp, t)
        check_scores(gemm["scores"][t, :n], I, A, f"scores t={t}")
        check_topk(gemm["idx"][t], int(gemm["count"][t]), I, A, inp.top_k, f"top-k t={t}")
