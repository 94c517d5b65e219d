"""csa_decode_step_noalloc (the decode step for callers that cannot allocate)
against csa_decode_step on the same inputs: every output bit-equal, on two
calls in a row, the second with a smaller input; and its size limit."""
import numpy as np
import pytest
import torch

from sparse_long_context_index_amd import inputs as gen
from tests._parity import say

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


def _run(inp, dev, noalloc, e4m3=False, one_sequence=False):
    b = B()
    d = b.upload(inp, dev)
    if e4m3:
        d = b.quantize_indexer_e4m3(d)
    outs = b.alloc_step_outputs(inp, dev)
    a = b.step_args(inp, d, outs, e4m3=e4m3, one_sequence=one_sequence)
    if noalloc:
        b.csa_decode_step_noalloc(a)
    else:
        # a workspace of non-zero bytes: the step must not rely on clear memory
        ws = torch.full((max(b.csa_decode_step_workspace_bytes(a), 1),), 0xA5, dtype=torch.uint8,
                        device=dev)
        b.csa_decode_step(a, ws)
    torch.cuda.synchronize(dev)
    return {k: v.cpu() for k, v in outs.items()}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (
        t.view(torch.int32) if t.dtype == torch.float32 else t)


def _same(x, y, what):
    assert x.keys() == y.keys()
    for k in x:
        assert torch.equal(_bits(x[k]), _bits(y[k])), f"{what}: {k} differs"
    assert int(x["err"][0]) == 0, f"{what}: device error"


def test_noalloc_matches_decode_step_twice_then_smaller(dev):
    say("csa_decode_step_noalloc: 1M step, then a 32K step, against csa_decode_step")
    big, small = gen.ctx1m(), gen.ctx32k()
    ref_big = _run(big, dev, False)
    ref_small = _run(small, dev, False)
    _same(_run(big, dev, True), ref_big, "1M")
    _same(_run(small, dev, True), ref_small, "32K after 1M")
    assert set(small.planted.tolist()) <= set(ref_small["idx"][0].tolist())


def test_noalloc_batched_and_e4m3(dev):
    say("csa_decode_step_noalloc: 32-sequence batch, then the tiny step with E4M3 keys")
    bat, tiny = gen.batched(), gen.tiny()
    _same(_run(bat, dev, True), _run(bat, dev, False), "batched")
    _same(_run(tiny, dev, True, e4m3=True), _run(tiny, dev, False, e4m3=True), "tiny E4M3")


def test_noalloc_gemm_indexer(dev):
    """The GEMM form of the indexer (640 tokens of one sequence, rows of about
    13,160 blocks, one_sequence set) through the allocation-free step."""
    say("csa_decode_step_noalloc: 640 tokens of one sequence, GEMM indexer")
    T = 640
    inp = gen.synth(11, pos=52000 + np.arange(T), seq_of_token=[0] * T,
                    n_comp_seq=[52000 // 4 + T // 4 + 1], n_ih=64, ihd=128, ratio=4, top_k=256,
                    window=64, n_heads=16, head_dim=128, w_std=0.125, swa_mode="per_token")
    _same(_run(inp, dev, True, one_sequence=True), _run(inp, dev, False, one_sequence=True),
          "GEMM indexer")


def test_noalloc_rejects_oversized_steps(dev):
    say("csa_decode_step_noalloc: a 4096-token prefill chunk needs more than the scratch")
    b = B()
    inp = gen.synth(9, pos=[65536 + i for i in range(64)], n_comp_seq=[16384], n_ih=64, ihd=128,
                    ratio=4, top_k=1024, window=128, n_heads=64, head_dim=512, w_std=0.125)
    d = b.upload(inp, dev)
    outs = b.alloc_step_outputs(inp, dev, max_vis=300000, keep=False)
    a = b.step_args(inp, d, outs, max_vis=300000)
    assert b.csa_decode_step_workspace_bytes(a) > b.CSA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(b.CSAError) as e:
        b.csa_decode_step_noalloc(a)
    assert e.value.status == b.CSA_ESCRATCH
    torch.cuda.synchronize(dev)
    assert int(outs["err"][0]) == 0  # nothing was launched
