"""The seeded input generators: bf16 rounding, determinism and layout."""
import numpy as np

from sparse_long_context_index_amd import inputs as gen


def test_bf16_round_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 1.0 + 2**-8 + 2**-20],
                 dtype=np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 ties up to 1+2^-6
    want = np.array([1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5, 1.0 + 2**-7], dtype=np.float32)
    np.testing.assert_array_equal(gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x)), want)


def test_workloads_deterministic_and_shaped():
    a, b = gen.tiny(), gen.tiny()
    for k in ("q_idx", "w", "k_idx", "comp_kv", "swa", "q"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    assert a.q_idx.shape == (1, 8, 32) and a.k_idx.shape == (63, 32)
    assert a.comp_kv.shape == (63, 64) and a.swa.shape == (16, 64) and a.q.shape == (1, 8, 64)
    assert a.max_visible() == 63 and a.scale == 0.125


def test_batched_layout():
    b = gen.batched()
    assert b.T == 32
    assert (b.n_comp == b.pos // 4).all()
    assert b.seq_kv[0] == 0 and (np.diff(b.seq_kv) == b.n_comp[:-1]).all()
    assert b.k_idx.shape[0] == int(b.n_comp.sum())
    assert (b.pos >= 16384).all() and (b.pos <= 131072).all()
    assert (b.swa_row0 == np.arange(32) * 128).all() and (b.swa_len == 128).all()


def test_prefill_linear_swa():
    p = gen.synth(4, pos=np.arange(1000, 1064), n_comp_seq=[256], n_ih=4, ihd=32, ratio=4,
                  top_k=16, window=8, n_heads=4, head_dim=64, w_std=0.5, swa_mode="linear")
    assert p.swa.shape[0] == 1063 - (1000 - 7) + 1
    assert (p.swa_row0 == np.arange(64)).all() and (p.swa_len == 8).all()
