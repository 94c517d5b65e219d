"""GPU parity of the producer side (csa_compress_append) against the CPU
oracle (oracle/producer_oracle.py).

* projections (the ring rows): |y_gpu - y_ref| <= 1e-4 * sum_k |x_k w_nk|;
* the sliding-window row and the pooled compressed rows (bf16):
  |v_gpu - v_ref| <= 2^-8 |v_ref| + 2e-3 * s, with s the largest |value|
  entering the row (the projection's own scale, or the largest |c| of the
  window's tokens in that channel), which covers the fp32 projection error
  carried into the softmax weights and one bf16 rounding;
* ring head and length, n_comp: exact.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_to_f64
from oracle import producer_oracle as P
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


def _bf(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def _dev_state(p, dev):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)  # noqa: E731
    return {"x": _bf(p.x, dev), "w_kv": _bf(p.w_kv, dev), "w_ik": _bf(p.w_ik, dev),
            "seq": t(p.seq, np.int32), "pos": t(p.pos, np.int64),
            "ring": t(p.ring, np.float32), "swa": _bf(p.swa, dev),
            "swa_head": t(p.swa_head, np.int32), "swa_len": t(p.swa_len, np.int32),
            "comp_kv": _bf(p.comp_kv, dev), "k_idx": _bf(p.k_idx, dev),
            "seq_kv": t(p.seq_kv, np.int64), "n_comp": t(p.n_comp, np.int32)}


def _run(p, d, dev):
    ws = torch.empty(max(B().csa_compress_append_workspace_bytes(p.T, p.H, p.hd, p.ihd), 1),
                     dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    B().csa_compress_append(d["x"], d["w_kv"], d["w_ik"], d["seq"], d["pos"], p.ratio, p.window,
                            d["ring"], d["swa"], d["swa_head"], d["swa_len"], d["comp_kv"],
                            d["k_idx"], d["seq_kv"], d["n_comp"], ws, err=err)
    torch.cuda.synchronize()
    return int(err.item())


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _close_bf16(got_bits, want, scale, what):
    got = bf16_to_f64(got_bits)
    bound = 2.0 ** -8 * np.abs(want) + 2e-3 * scale + 1e-30
    bad = np.nonzero(np.abs(got - want) > bound)
    assert bad[0].size == 0, f"{what}: {bad[0].size} values out of tolerance, first {bad[0][:4]}"


def _check(p, d, st, out):
    """GPU state d (after the call) against the oracle state st (after the
    same step) and its fp64 intermediates."""
    y = out["y"]
    x = bf16_to_f64(p.x)
    W = np.concatenate([bf16_to_f64(p.w_kv), bf16_to_f64(p.w_ik)])
    Y = np.abs(x) @ np.abs(W).T                        # sum_k |x_k w_nk|
    ring = d["ring"].cpu().numpy().astype(np.float64)
    R = 2 * p.ratio
    for t in range(p.T):
        s, q = int(p.seq[t]), int(p.pos[t])
        err = np.abs(ring[s, q % R] - y[t])
        assert (err <= 1e-4 * Y[t] + 1e-30).all(), f"ring row of token {t}: max {err.max()}"
    # untouched ring rows are unchanged
    touched = {(int(p.seq[t]), int(p.pos[t]) % R) for t in range(p.T)}
    for s in range(ring.shape[0]):
        for r in range(R):
            if (s, r) not in touched:
                assert np.array_equal(ring[s, r], p.ring[s, r].astype(np.float64))
    assert np.array_equal(d["swa_head"].cpu().numpy(), st.swa_head)
    assert np.array_equal(d["swa_len"].cpu().numpy(), st.swa_len)
    assert np.array_equal(d["n_comp"].cpu().numpy(), st.n_comp)
    swa = _bits(d["swa"])
    for t in range(p.T):
        s = int(p.seq[t])
        h = int(p.swa_head[s])
        _close_bf16(swa[s, h], y[t, :p.hd], Y[t, :p.hd], f"window row of token {t}")
        others = [k for k in range(p.window) if k != h]
        assert np.array_equal(swa[s, others], p.swa[s, others])
    ck, ki = _bits(d["comp_kv"]), _bits(d["k_idx"])
    written = set()
    for t, (e_kv, e_ik, rows) in out["pooled"].items():
        s = int(p.seq[t])
        i = (int(p.pos[t]) + 1) // p.ratio - 1
        r = int(p.seq_kv[s]) + i
        written.add(r)
        hd, ihd = p.hd, p.ihd
        _close_bf16(ck[r], e_kv, np.abs(rows[:, :hd]).max(axis=0), f"comp_kv row of token {t}")
        _close_bf16(ki[r], e_ik, np.abs(rows[:, 2 * hd:2 * hd + ihd]).max(axis=0),
                    f"k_idx row of token {t}")
    for r in range(ck.shape[0]):
        if r not in written:
            assert np.array_equal(ck[r], p.comp_kv[r]) and np.array_equal(ki[r], p.k_idx[r])
    return len(written)


def _oracle_step(p):
    st = P.ProducerState(ring=p.ring.astype(np.float64), swa=p.swa, swa_head=p.swa_head,
                         swa_len=p.swa_len, comp_kv=p.comp_kv, k_idx=p.k_idx, seq_kv=p.seq_kv,
                         n_comp=p.n_comp)
    out = P.append_step(st, p.x, p.seq, p.pos, p.w_kv, p.w_ik, p.hd, p.ihd, p.ratio, p.window)
    return st, out


@pytest.mark.parametrize("T", [1, 32])
def test_compress_append_1m_shape(dev, T):
    say(f"csa_compress_append H 7168, hd 512, ihd 128, ratio 4, window 128, {T} tokens")
    p = gen.producer_1m(T=T)
    # make sure both branches occur: token 0 ends a block, token 1 does not
    p.pos[0] = p.pos[0] - p.pos[0] % p.ratio + p.ratio - 1
    p.n_comp[p.seq[0]] = p.pos[0] // p.ratio
    p.seq_kv[p.seq[0]] = 2 * p.seq[0] + 1 - p.n_comp[p.seq[0]]
    p.swa_head[p.seq[0]] = p.pos[0] % p.window
    if T > 1:
        if (p.pos[1] + 1) % p.ratio == 0:
            p.pos[1] -= 1
            p.n_comp[p.seq[1]] = p.pos[1] // p.ratio
            p.seq_kv[p.seq[1]] = 2 * p.seq[1] + 1 - p.n_comp[p.seq[1]]
        p.swa_head[p.seq[:2]] = (p.pos[:2] % p.window).astype(np.int32)
    d = _dev_state(p, dev)
    assert _run(p, d, dev) == 0
    st, out = _oracle_step(p)
    n = _check(p, d, st, out)
    say(f"  blocks completed: {n}")
    assert n >= 1 and (T == 1 or len(out["pooled"]) < T)


@pytest.mark.parametrize("ratio", [1, 2, 4, 16])
def test_compress_append_sequence_of_steps(dev, ratio):
    say(f"csa_compress_append: 3 sequences, 21 decode steps each, ratio {ratio}, small shapes")
    S, H, hd, ihd, window = 3, 256, 16, 32, 8
    p = gen.producer(11, S=S, T=S, H=H, hd=hd, ihd=ihd, ratio=ratio, window=window, max_pos=1)
    # fresh sequences at positions 0, 1, 2; empty rings; room for 8 blocks each
    p.ring[:] = 0.0
    p.swa[:] = 0
    p.swa_head[:] = [0, 1, 2]
    p.swa_len[:] = [0, 1, 2]
    p.n_comp[:] = np.array([0, 1, 2]) // ratio   # the blocks the earlier tokens completed
    rows = 32
    p.seq_kv[:] = np.arange(S) * rows
    p.comp_kv = np.zeros((S * rows, hd), np.uint16)
    p.k_idx = np.zeros((S * rows, ihd), np.uint16)
    start = np.array([0, 1, 2])
    d = _dev_state(p, dev)
    r = np.random.default_rng(12)
    for step in range(21):
        p.pos = (start + step).astype(np.int64)
        p.seq = np.arange(S, dtype=np.int32)
        p.x = gen.f32_to_bf16_bits(r.standard_normal((S, H)).astype(np.float32))
        d["x"], d["pos"] = _bf(p.x, dev), torch.from_numpy(p.pos).to(dev)
        d["seq"] = torch.from_numpy(p.seq).to(dev)
        assert _run(p, d, dev) == 0
        st, out = _oracle_step(p)
        _check(p, d, st, out)
        # carry the GPU's state forward on both sides (the oracle starts each
        # step from the GPU's ring, window and caches)
        p.ring = d["ring"].cpu().numpy()
        p.swa = _bits(d["swa"])
        p.swa_head = d["swa_head"].cpu().numpy()
        p.swa_len = d["swa_len"].cpu().numpy()
        p.n_comp = d["n_comp"].cpu().numpy()
        p.comp_kv, p.k_idx = _bits(d["comp_kv"]), _bits(d["k_idx"])
    assert p.n_comp.tolist() == [(int(s0) + 21) // ratio for s0 in start]  # 21, 22, 23 tokens seen
    assert p.swa_len.tolist() == [8, 8, 8]


def test_compress_append_flags_bad_rows(dev):
    say("csa_compress_append: a compressed row outside the cache is flagged, not written")
    p = gen.producer(13, S=2, T=1, H=256, hd=16, ihd=16, ratio=4, window=8, max_pos=64)
    p.pos[0] = 4 * (p.pos[0] // 4) + 3
    s = int(p.seq[0])
    p.n_comp[s] = p.pos[0] // 4
    p.seq_kv[s] = 100                                      # beyond the 4 rows
    d = _dev_state(p, dev)
    before = (_bits(d["comp_kv"]).copy(), _bits(d["k_idx"]).copy())
    e = _run(p, d, dev)
    assert e & 0x2, f"{e:#x}"                              # CSA_DERR_KEY_RANGE
    assert np.array_equal(_bits(d["comp_kv"]), before[0])
    assert np.array_equal(_bits(d["k_idx"]), before[1])
