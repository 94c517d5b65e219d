"""libcsa on the host: it loads, exports every entry point that include/csa.h
declares, and rejects bad arguments with the documented status before any
GPU work (every call below fails validation or is a T == 0 no-op, so no
kernel is launched and no device memory is touched)."""
import ctypes
import os
import re

import pytest

from sparse_long_context_index_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 256-byte aligned non-null address; never dereferenced here


def _header_functions():
    text = open(os.path.join(ROOT, "include", "csa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return b.load()


def test_exports_every_declared_symbol(lib):
    names = _header_functions()
    assert len(names) == 16, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(b.EXPORTS)


def test_status_strings_and_version(lib):
    assert b.csa_abi_version() == 3
    assert b.csa_status_str(0) == "CSA_OK"
    for s in (1, 2, 3, 4):
        assert b.csa_status_str(s).startswith("CSA_E")
    assert "unknown" in b.csa_status_str(99)


def _index(lib, **kw):
    a = dict(q_idx=FAKE, w=FAKE, k_idx=FAKE, k_rows=100, pos=FAKE, seq_kv=FAKE, n_comp=FAKE,
             T=1, n_ih=64, ihd=128, ratio=4, scores=FAKE, ld=100, err=None, stream=None)
    a.update(kw)
    return lib.csa_index_score(*a.values())


def test_index_score_e4m3_and_quantize_validation(lib):
    a = dict(q_idx=FAKE, q_scale=FAKE, w=FAKE, k_idx=FAKE, k_scale=FAKE, k_rows=100, pos=FAKE,
             seq_kv=FAKE, n_comp=FAKE, T=1, n_ih=64, ihd=128, ratio=4, scores=FAKE, ld=100,
             err=None, stream=None)
    f = lambda **kw: lib.csa_index_score_e4m3(*dict(a, **kw).values())  # noqa: E731
    assert f(T=0) == b.CSA_OK
    assert f(q_scale=None) == b.CSA_EINVAL
    assert f(k_scale=None) == b.CSA_EINVAL
    assert f(k_idx=FAKE + 8) == b.CSA_EINVAL                 # codes must be 16-byte aligned
    assert f(ihd=48) == b.CSA_EUNSUPPORTED
    q = lambda **kw: lib.csa_quantize_e4m3(*dict(dict(src=FAKE, rows=10, d=128, codes=FAKE,  # noqa: E731
                                                      scale=FAKE, stream=None), **kw).values())
    assert q(rows=0) == b.CSA_OK
    assert q(d=0) == b.CSA_EINVAL
    assert q(d=513) == b.CSA_EUNSUPPORTED
    assert q(codes=None) == b.CSA_EINVAL
    assert q(rows=-1) == b.CSA_EINVAL


def test_index_score_validation(lib):
    assert _index(lib, T=0) == b.CSA_OK                      # no-op
    assert _index(lib, q_idx=None) == b.CSA_EINVAL
    assert _index(lib, scores=None) == b.CSA_EINVAL
    assert _index(lib, ihd=48) == b.CSA_EUNSUPPORTED
    assert _index(lib, n_ih=0) == b.CSA_EINVAL
    assert _index(lib, n_ih=129) == b.CSA_EUNSUPPORTED
    assert _index(lib, ratio=0) == b.CSA_EINVAL
    assert _index(lib, ld=0) == b.CSA_EINVAL
    assert _index(lib, T=-1) == b.CSA_EINVAL
    assert _index(lib, q_idx=FAKE + 2) == b.CSA_EINVAL      # misaligned bf16 tensor
    assert _index(lib, T=70000) == b.CSA_EUNSUPPORTED


def test_topk_validation(lib):
    # a row longer than the LDS pool needs candidate lists in the workspace
    ld = 100000
    args = lambda **kw: {**dict(scores=FAKE, ld=ld, pos=FAKE, n_comp=FAKE, T=1, ratio=4,  # noqa
                                top_k=16, idx=FAKE, count=FAKE, ws=FAKE, ws_bytes=1 << 30,
                                err=None, stream=None), **kw}
    f = lambda **kw: lib.csa_topk(*args(**kw).values())  # noqa: E731
    assert f(T=0) == b.CSA_OK
    assert f(top_k=0) == b.CSA_EINVAL
    assert f(top_k=2049) == b.CSA_EUNSUPPORTED
    assert f(idx=None) == b.CSA_EINVAL
    assert f(ws=None) == b.CSA_EWORKSPACE
    assert f(ws=FAKE + 16) == b.CSA_EWORKSPACE               # not 256-byte aligned
    need = b.csa_topk_workspace_bytes(1, ld, 16)
    assert need > 0
    assert f(ws_bytes=need - 1) == b.CSA_EWORKSPACE
    # rows that fit the LDS pool select straight from the scores: no workspace
    assert b.csa_topk_workspace_bytes(4, 12288, 1024) == 0


def test_gather_validation(lib):
    base = dict(comp_kv=FAKE, comp_rows=10, seq_kv=FAKE, idx=FAKE, count=FAKE, top_k=16,
                swa=FAKE, swa_rows=16, swa_row0=FAKE, swa_len=FAKE, window=16, T=1,
                head_dim=64, all_kv=FAKE, n_kv=FAKE, err=None, stream=None)
    f = lambda **kw: lib.csa_gather(*{**base, **kw}.values())  # noqa: E731
    assert f(T=0) == b.CSA_OK
    assert f(head_dim=96) == b.CSA_EUNSUPPORTED
    assert f(all_kv=None) == b.CSA_EINVAL
    assert f(window=-1) == b.CSA_EINVAL
    assert f(top_k=4096) == b.CSA_EUNSUPPORTED


def test_attend_validation(lib):
    base = dict(q=FAKE, T=1, n_heads=8, head_dim=64, scale=0.125, sink=None, kv_a=FAKE,
                a_rows=100, a_row0=FAKE, a_len=FAKE, kv_b=None, b_rows=0, b_row0=None,
                b_len=None, max_rows=100, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30,
                err=None, stream=None)
    f = lambda **kw: lib.csa_mqa_attend(*{**base, **kw}.values())  # noqa: E731
    assert f(T=0) == b.CSA_OK
    assert f(head_dim=80) == b.CSA_EUNSUPPORTED
    assert f(n_heads=0) == b.CSA_EINVAL
    assert f(n_heads=129) == b.CSA_EUNSUPPORTED
    assert f(kv_b=FAKE) == b.CSA_EINVAL                        # partial second segment
    assert f(scale=float("nan")) == b.CSA_EINVAL
    assert f(a_len=None) == b.CSA_EINVAL
    big = b.csa_attend_workspace_bytes(1, 64, 512, 100000)
    assert f(head_dim=512, n_heads=64, max_rows=100000, ws_bytes=big - 1) == b.CSA_EWORKSPACE


def test_decode_step_validation(lib):
    a = b.StepArgs()
    a.mode, a.T, a.n_ih, a.ihd, a.ratio, a.top_k, a.window = 0, 1, 64, 128, 4, 1024, 128
    a.n_heads, a.head_dim, a.max_vis, a.scale = 64, 512, 262144, 0.0441941738
    for k in ("q_idx", "w", "k_idx", "comp_kv", "swa", "q", "pos", "seq_kv", "n_comp",
              "swa_row0", "swa_len", "all_kv", "out"):
        setattr(a, k, FAKE)
    a.k_rows = a.comp_rows = 262144
    a.swa_rows = 128
    need = b.csa_decode_step_workspace_bytes(a)
    # at least the scores of 262,144 blocks plus the attention split partials
    assert need >= 262144 * 4 + 64 * 512 * 4
    st = lambda ws, n: lib.csa_decode_step(ctypes.byref(a), ws, n, None)  # noqa: E731
    assert st(None, 0) == b.CSA_EWORKSPACE
    assert st(FAKE, need - 1) == b.CSA_EWORKSPACE
    a.mode = 7
    assert st(FAKE, need) == b.CSA_EINVAL
    a.mode = 0
    a.top_k = 0
    assert st(FAKE, need) == b.CSA_EINVAL
    a.top_k = 1024
    a.all_kv = FAKE + 2  # all_kv is optional, but must be 16-byte aligned when given
    assert st(FAKE, need) == b.CSA_EINVAL
    a.all_kv = None
    assert b.csa_decode_step_workspace_bytes(a) == need
    a.all_kv = FAKE
    a.idx_e4m3 = 1                # the E4M3 prefilter needs the codes and both scale arrays
    assert st(FAKE, need) == b.CSA_EINVAL
    a.q_idx_scale = a.k_idx_scale = FAKE
    assert st(FAKE, need) == b.CSA_EINVAL
    a.q_idx8 = a.k_idx8 = FAKE
    need8 = b.csa_decode_step_workspace_bytes(a)
    # prefilter of C = 1536 candidates: indices, count, keys and a bound per token
    assert need8 > need
    assert need8 - need >= 1536 * 12
    assert st(FAKE, need) == b.CSA_EWORKSPACE
    a.k_idx8 = FAKE + 8           # codes are read 16 bytes at a time
    assert st(FAKE, need8) == b.CSA_EINVAL
    a.idx_e4m3 = 0
    a.k_idx8 = FAKE
    a.one_sequence = 2            # a flag: 0 or 1
    assert st(FAKE, need) == b.CSA_EINVAL
    a.one_sequence = 1            # no workspace of its own
    assert b.csa_decode_step_workspace_bytes(a) == need
    a.k_idx8 = FAKE
    a.idx_e4m3 = 2
    assert st(FAKE, need8) == b.CSA_EINVAL
    a.idx_e4m3 = 0
    a.head_dim = 100
    assert st(FAKE, need) == b.CSA_EUNSUPPORTED
    a.head_dim = 512
    # the allocation-free step refuses, before touching a GPU, a step whose
    # workspace would not fit its fixed scratch (here 1 GiB of scores)
    a.max_vis = 1 << 28
    assert b.csa_decode_step_workspace_bytes(a) > b.CSA_NOALLOC_SCRATCH_BYTES
    assert lib.csa_decode_step_noalloc(ctypes.byref(a), None) == b.CSA_ESCRATCH
    assert "CSA_NOALLOC_SCRATCH_BYTES" in b.csa_status_str(b.CSA_ESCRATCH)
    a.max_vis = 262144
    stage = lambda k, ws, n: lib.csa_decode_step_stage(ctypes.byref(a), k, ws, n, None)  # noqa: E731
    assert stage(0, FAKE, need) == b.CSA_EINVAL and stage(3, FAKE, need) == b.CSA_EINVAL
    assert stage(b.CSA_STAGE_INDEX, FAKE, need - 1) == b.CSA_EWORKSPACE
    assert stage(b.CSA_STAGE_REST, None, 0) == b.CSA_EWORKSPACE
    a.T = 0
    assert st(FAKE, need) == b.CSA_OK
    assert lib.csa_decode_step_noalloc(ctypes.byref(a), None) == b.CSA_OK
    assert lib.csa_decode_step(None, FAKE, need, None) == b.CSA_EINVAL


def test_binding_refuses_cpu_tensors():
    import torch
    t = torch.zeros(4, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        b._p(t, (torch.float32,), "x")


def test_compress_append_validation(lib):
    f = lambda **kw: lib.csa_compress_append(*{**dict(  # noqa: E731
        x=FAKE, T=1, H=7168, w_kv=FAKE, hd=512, w_ik=FAKE, ihd=128, seq=FAKE, pos=FAKE, S=4,
        ratio=4, window=128, ring=FAKE, swa=FAKE, swa_head=FAKE, swa_len=FAKE, comp_kv=FAKE,
        k_idx=FAKE, seq_kv=FAKE, n_comp=FAKE, comp_rows=8, ws=FAKE, ws_bytes=1 << 24,
        err=None, stream=None), **kw}.values())
    need = b.csa_compress_append_workspace_bytes(1, 7168, 512, 128)
    # split-K partials: 7 chunks of 1024 x (2*512 + 2*128) fp32 for one token
    assert need == 7 * 1280 * 4
    assert f(T=0) == b.CSA_OK
    assert f(x=None) == b.CSA_EINVAL
    assert f(x=FAKE + 8) == b.CSA_EINVAL          # 16-byte loads of x rows
    assert f(H=7000) == b.CSA_EUNSUPPORTED        # not a multiple of 256
    assert f(hd=520) == b.CSA_EUNSUPPORTED
    assert f(ratio=32) == b.CSA_EUNSUPPORTED and f(ratio=3) == b.CSA_EUNSUPPORTED
    assert f(S=0) == b.CSA_EINVAL
    assert f(ws_bytes=need - 1) == b.CSA_EWORKSPACE
    assert f(ws=FAKE + 16) == b.CSA_EWORKSPACE

