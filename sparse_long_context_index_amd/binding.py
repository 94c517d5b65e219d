"""ctypes binding of libcsa (include/csa.h).

Argument marshalling only: every function checks that the torch tensors it is
given live on the GPU, are contiguous and have the expected dtype, then passes
their device pointers and the current HIP stream to the C entry point of the
same name.  Nothing here computes any part of the method, and there is no CPU
fallback: if libcsa.so is missing or a call fails, an exception is raised.

bf16 tensors may be torch.bfloat16, torch.int16 or torch.uint16 (bit patterns).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
_lib = None

CSA_OK, CSA_EINVAL, CSA_EUNSUPPORTED, CSA_EWORKSPACE, CSA_EHIP, CSA_ESCRATCH = range(6)
CSA_NOALLOC_SCRATCH_BYTES = 64 << 20
CSA_STAGE_INDEX, CSA_STAGE_REST = 1, 2
CSA_MODE_CSA, CSA_MODE_HCA = 0, 1
DERR = {0x1: "VIS_OVER_LD", 0x2: "KEY_RANGE", 0x4: "BAD_META", 0x8: "ROW_RANGE",
        0x10: "COUNT_RANGE", 0x20: "ROWS_OVER_MAX"}

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class CSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {csa_status_str(status)} ({status})")
        self.status = status


class StepArgs(ctypes.Structure):
    """Mirror of csa_step_args."""
    _fields_ = [
        ("mode", _i32), ("T", _i32), ("n_ih", _i32), ("ihd", _i32), ("ratio", _i32),
        ("top_k", _i32), ("window", _i32), ("n_heads", _i32), ("head_dim", _i32),
        ("max_vis", _i64), ("scale", _f32),
        ("q_idx", _vp), ("w", _vp), ("k_idx", _vp), ("k_rows", _i64),
        ("comp_kv", _vp), ("comp_rows", _i64), ("swa", _vp), ("swa_rows", _i64),
        ("q", _vp), ("sink", _vp), ("pos", _vp), ("seq_kv", _vp), ("n_comp", _vp),
        ("swa_row0", _vp), ("swa_len", _vp), ("all_kv", _vp), ("out", _vp), ("lse", _vp),
        ("scores", _vp), ("idx", _vp), ("count", _vp), ("n_kv", _vp), ("err", _vp),
        ("idx_e4m3", _i32), ("q_idx8", _vp), ("q_idx_scale", _vp), ("k_idx8", _vp),
        ("k_idx_scale", _vp), ("one_sequence", _i32),
    ]


_SIGS = {
    "csa_status_str": (ctypes.c_char_p, [_i32]),
    "csa_abi_version": (_i32, []),
    "csa_index_score": (_i32, [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                               _vp, _i64, _vp, _vp]),
    "csa_index_score_e4m3": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32,
                                    _i32, _i32, _vp, _i64, _vp, _vp]),
    "csa_quantize_e4m3": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp]),
    "csa_topk_workspace_bytes": (_sz, [_i32, _i64, _i32]),
    "csa_topk": (_i32, [_vp, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp, _vp]),
    "csa_gather": (_i32, [_vp, _i64, _vp, _vp, _vp, _i32, _vp, _i64, _vp, _vp, _i32, _i32, _i32,
                          _vp, _vp, _vp, _vp]),
    "csa_attend_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "csa_mqa_attend": (_i32, [_vp, _i32, _i32, _i32, _f32, _vp, _vp, _i64, _vp, _vp, _vp, _i64,
                              _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp, _vp]),
    "csa_decode_step_workspace_bytes": (_sz, [ctypes.POINTER(StepArgs)]),
    "csa_decode_step": (_i32, [ctypes.POINTER(StepArgs), _vp, _sz, _vp]),
    "csa_decode_step_noalloc": (_i32, [ctypes.POINTER(StepArgs), _vp]),
    "csa_compress_append_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "csa_compress_append": (_i32, [_vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32,
                                   _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _sz,
                                   _vp, _vp]),
    "csa_decode_step_stage": (_i32, [ctypes.POINTER(StepArgs), _i32, _vp, _sz, _vp]),
}
EXPORTS = tuple(_SIGS)


def load(reload: bool = False):
    """Load libcsa.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None and not reload:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def csa_status_str(status: int) -> str:
    return load().csa_status_str(status).decode()


def csa_abi_version() -> int:
    return load().csa_abi_version()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _p(t: Optional[torch.Tensor], dtypes, name: str, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (the library has no CPU path)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(fn: str, status: int):
    if status != CSA_OK:
        raise CSAError(fn, status)


def csa_index_score(q_idx, w, k_idx, pos, seq_kv, n_comp, n_ih, ihd, ratio, scores, ld,
                    err=None, stream=None):
    T = int(pos.shape[0])
    _check("csa_index_score", load().csa_index_score(
        _p(q_idx, _BF16, "q_idx"), _p(w, (torch.float32,), "w"), _p(k_idx, _BF16, "k_idx"),
        int(k_idx.shape[0]), _p(pos, (torch.int64,), "pos"), _p(seq_kv, (torch.int64,), "seq_kv"),
        _p(n_comp, (torch.int32,), "n_comp"), T, n_ih, ihd, ratio,
        _p(scores, (torch.float32,), "scores"), ld, _p(err, (torch.int32,), "err", True),
        _stream(stream)))


def csa_index_score_e4m3(q_idx, q_scale, w, k_idx, k_scale, pos, seq_kv, n_comp, n_ih, ihd,
                         ratio, scores, ld, err=None, stream=None):
    T = int(pos.shape[0])
    _check("csa_index_score_e4m3", load().csa_index_score_e4m3(
        _p(q_idx, (torch.uint8,), "q_idx"), _p(q_scale, (torch.float32,), "q_scale"),
        _p(w, (torch.float32,), "w"), _p(k_idx, (torch.uint8,), "k_idx"),
        _p(k_scale, (torch.float32,), "k_scale"), int(k_idx.shape[0]),
        _p(pos, (torch.int64,), "pos"), _p(seq_kv, (torch.int64,), "seq_kv"),
        _p(n_comp, (torch.int32,), "n_comp"), T, n_ih, ihd, ratio,
        _p(scores, (torch.float32,), "scores"), ld,
        _p(err, (torch.int32, torch.uint32), "err", optional=True), _stream(stream)))


def csa_quantize_e4m3(src, codes, scale, stream=None):
    """src [rows, d] bf16 -> codes [rows, d] uint8 (E4M3), scale [rows] fp32."""
    rows, d = int(src.shape[0]), int(src.shape[1]) if src.dim() > 1 else 1
    _check("csa_quantize_e4m3", load().csa_quantize_e4m3(
        _p(src, _BF16, "src"), rows, d, _p(codes, (torch.uint8,), "codes"),
        _p(scale, (torch.float32,), "scale"), _stream(stream)))


def csa_topk_workspace_bytes(T, ld, top_k) -> int:
    return int(load().csa_topk_workspace_bytes(T, ld, top_k))


def csa_topk(scores, ld, pos, n_comp, ratio, top_k, idx, count, ws, err=None, stream=None):
    T = int(pos.shape[0])
    _check("csa_topk", load().csa_topk(
        _p(scores, (torch.float32,), "scores"), ld, _p(pos, (torch.int64,), "pos"),
        _p(n_comp, (torch.int32,), "n_comp"), T, ratio, top_k, _p(idx, (torch.int32,), "idx"),
        _p(count, (torch.int32,), "count"), _p(ws, (torch.uint8,), "ws", True),
        0 if ws is None else ws.numel(), _p(err, (torch.int32,), "err", True), _stream(stream)))


def csa_gather(comp_kv, seq_kv, idx, count, top_k, swa, swa_row0, swa_len, window, head_dim,
               all_kv, n_kv, err=None, stream=None):
    T = int(seq_kv.shape[0])
    _check("csa_gather", load().csa_gather(
        _p(comp_kv, _BF16, "comp_kv"), int(comp_kv.shape[0]), _p(seq_kv, (torch.int64,), "seq_kv"),
        _p(idx, (torch.int32,), "idx"), _p(count, (torch.int32,), "count"), top_k,
        _p(swa, _BF16, "swa"), int(swa.shape[0]), _p(swa_row0, (torch.int64,), "swa_row0"),
        _p(swa_len, (torch.int32,), "swa_len"), window, T, head_dim, _p(all_kv, _BF16, "all_kv"),
        _p(n_kv, (torch.int32,), "n_kv"), _p(err, (torch.int32,), "err", True), _stream(stream)))


def csa_attend_workspace_bytes(T, n_heads, head_dim, max_rows) -> int:
    return int(load().csa_attend_workspace_bytes(T, n_heads, head_dim, max_rows))


def csa_mqa_attend(q, n_heads, head_dim, scale, kv_a, a_row0, a_len, max_rows, out,
                   kv_b=None, b_row0=None, b_len=None, sink=None, lse=None, ws=None,
                   err=None, stream=None):
    T = int(a_row0.shape[0])
    _check("csa_mqa_attend", load().csa_mqa_attend(
        _p(q, _BF16, "q"), T, n_heads, head_dim, float(scale),
        _p(sink, (torch.float32,), "sink", True), _p(kv_a, _BF16, "kv_a"), int(kv_a.shape[0]),
        _p(a_row0, (torch.int64,), "a_row0"), _p(a_len, (torch.int32,), "a_len"),
        _p(kv_b, _BF16, "kv_b", True), 0 if kv_b is None else int(kv_b.shape[0]),
        _p(b_row0, (torch.int64,), "b_row0", True), _p(b_len, (torch.int32,), "b_len", True),
        max_rows, _p(out, _BF16, "out"), _p(lse, (torch.float32,), "lse", True),
        _p(ws, (torch.uint8,), "ws", True), 0 if ws is None else ws.numel(),
        _p(err, (torch.int32,), "err", True), _stream(stream)))


def csa_decode_step_workspace_bytes(args: StepArgs) -> int:
    return int(load().csa_decode_step_workspace_bytes(ctypes.byref(args)))


def step_workspace(args: StepArgs, dev) -> "torch.Tensor":
    """A decode-step workspace of the size the C ABI asks for (its contents
    on entry do not matter; it is zero-filled here only for reproducibility)."""
    import torch
    return torch.zeros(max(csa_decode_step_workspace_bytes(args), 1), dtype=torch.uint8, device=dev)


def csa_decode_step(args: StepArgs, ws, stream=None):
    _check("csa_decode_step", load().csa_decode_step(
        ctypes.byref(args), _p(ws, (torch.uint8,), "ws", True), 0 if ws is None else ws.numel(),
        _stream(stream)))


def csa_decode_step_stage(args: StepArgs, stage: int, ws, stream=None):
    _check("csa_decode_step_stage", load().csa_decode_step_stage(
        ctypes.byref(args), int(stage), _p(ws, (torch.uint8,), "ws", True),
        0 if ws is None else ws.numel(), _stream(stream)))


def csa_compress_append_workspace_bytes(T, H, hd, ihd) -> int:
    return int(load().csa_compress_append_workspace_bytes(T, H, hd, ihd))


def csa_compress_append(x, w_kv, w_ik, seq, pos, ratio, window, ring, swa, swa_head, swa_len,
                        comp_kv, k_idx, seq_kv, n_comp, ws, err=None, stream=None):
    """x [T, H] bf16; w_kv [2hd, H], w_ik [2ihd, H] bf16; ring [S, 2*ratio,
    2hd + 2ihd] fp32; swa [S, window, hd] bf16; comp_kv [rows, hd], k_idx
    [rows, ihd] bf16; per sequence swa_head, swa_len, n_comp int32, seq_kv
    int64; per token seq int32, pos int64."""
    T, H = int(x.shape[0]), int(x.shape[1])
    hd, ihd, S = int(w_kv.shape[0]) // 2, int(w_ik.shape[0]) // 2, int(ring.shape[0])
    _check("csa_compress_append", load().csa_compress_append(
        _p(x, _BF16, "x"), T, H, _p(w_kv, _BF16, "w_kv"), hd, _p(w_ik, _BF16, "w_ik"), ihd,
        _p(seq, (torch.int32,), "seq"), _p(pos, (torch.int64,), "pos"), S, ratio, window,
        _p(ring, (torch.float32,), "ring"), _p(swa, _BF16, "swa"),
        _p(swa_head, (torch.int32,), "swa_head"), _p(swa_len, (torch.int32,), "swa_len"),
        _p(comp_kv, _BF16, "comp_kv"), _p(k_idx, _BF16, "k_idx"),
        _p(seq_kv, (torch.int64,), "seq_kv"), _p(n_comp, (torch.int32,), "n_comp"),
        int(comp_kv.shape[0]), _p(ws, (torch.uint8,), "ws", True), 0 if ws is None else ws.numel(),
        _p(err, (torch.int32, torch.uint32), "err", optional=True), _stream(stream)))


def csa_decode_step_noalloc(args: StepArgs, stream=None):
    """csa_decode_step with the library's fixed per-GPU scratch as workspace."""
    _check("csa_decode_step_noalloc",
           load().csa_decode_step_noalloc(ctypes.byref(args), _stream(stream)))


# ---------------------------------------------------------------------------
# Marshalling helpers for the synthetic workloads (upload, argument packing).
# ---------------------------------------------------------------------------

def _bf16_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def upload(inp, dev) -> dict:
    """Copy a CSAInputs batch to the device (bf16 as torch.bfloat16)."""
    d = {}
    for k in ("q_idx", "k_idx", "comp_kv", "swa", "q"):
        d[k] = _bf16_dev(getattr(inp, k), dev)
    d["w"] = torch.from_numpy(np.ascontiguousarray(inp.w)).to(dev)
    for k in ("pos", "seq_kv", "swa_row0"):
        d[k] = torch.from_numpy(np.ascontiguousarray(getattr(inp, k), dtype=np.int64)).to(dev)
    for k in ("n_comp", "swa_len"):
        d[k] = torch.from_numpy(np.ascontiguousarray(getattr(inp, k), dtype=np.int32)).to(dev)
    return d


def quantize_indexer_e4m3(d: dict, stream=None) -> dict:
    """E4M3 codes and scales of the uploaded indexer queries and keys, made on
    the GPU by csa_quantize_e4m3 (q_idx8, q_scale [T, n_ih], k_idx8, k_scale)."""
    q, k = d["q_idx"], d["k_idx"]
    T, n_ih, ihd = q.shape
    q8 = torch.empty((T, n_ih, ihd), dtype=torch.uint8, device=q.device)
    qs = torch.empty((T, n_ih), dtype=torch.float32, device=q.device)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=k.device)
    ks = torch.empty(k.shape[0], dtype=torch.float32, device=k.device)
    csa_quantize_e4m3(q.reshape(T * n_ih, ihd), q8.view(T * n_ih, ihd), qs.view(-1), stream)
    csa_quantize_e4m3(k, k8, ks, stream)
    d = dict(d)
    d.update(q_idx8=q8, q_scale=qs, k_idx8=k8, k_scale=ks)
    return d


def step_args(inp, d: dict, outs: dict, mode: int = CSA_MODE_CSA, max_vis: Optional[int] = None,
              sink: Optional[torch.Tensor] = None, e4m3: bool = False,
              one_sequence: bool = False) -> StepArgs:
    """Pack a csa_step_args for a CSAInputs batch whose tensors are in `d`
    (see upload) and whose outputs are in `outs` (all_kv, out, lse, scores,
    idx, count, n_kv, err; any may be absent).  one_sequence: the caller's
    promise that every token's key rows start at the same seq_kv."""
    a = StepArgs()
    a.mode = mode
    a.T, a.n_ih, a.ihd, a.ratio = inp.T, inp.n_ih, inp.ihd, inp.ratio
    a.top_k, a.window, a.n_heads, a.head_dim = inp.top_k, inp.window, inp.n_heads, inp.head_dim
    a.max_vis = int(max_vis if max_vis is not None else max(inp.max_visible(), 1))
    a.scale = float(inp.scale)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    a.q_idx, a.w, a.k_idx = ptr(d["q_idx"]), ptr(d["w"]), ptr(d["k_idx"])
    a.k_rows = int(d["k_idx"].shape[0])
    a.comp_kv, a.comp_rows = ptr(d["comp_kv"]), int(d["comp_kv"].shape[0])
    a.swa, a.swa_rows = ptr(d["swa"]), int(d["swa"].shape[0])
    a.q, a.sink = ptr(d["q"]), ptr(sink)
    a.pos, a.seq_kv, a.n_comp = ptr(d["pos"]), ptr(d["seq_kv"]), ptr(d["n_comp"])
    a.swa_row0, a.swa_len = ptr(d["swa_row0"]), ptr(d["swa_len"])
    for k in ("all_kv", "out", "lse", "scores", "idx", "count", "n_kv", "err"):
        setattr(a, k, ptr(outs.get(k)))
    if e4m3:
        a.idx_e4m3 = 1
        a.q_idx8, a.k_idx8 = ptr(d["q_idx8"]), ptr(d["k_idx8"])
        a.q_idx_scale, a.k_idx_scale = ptr(d["q_scale"]), ptr(d["k_scale"])
    a.one_sequence = 1 if one_sequence else 0
    return a


def alloc_step_outputs(inp, dev, max_vis: Optional[int] = None, keep=True,
                       all_kv=True) -> dict:
    mv = int(max_vis if max_vis is not None else max(inp.max_visible(), 1))
    T = inp.T
    o = {
        "out": torch.zeros((T, inp.n_heads, inp.head_dim), dtype=torch.bfloat16, device=dev),
        "lse": torch.zeros((T, inp.n_heads), dtype=torch.float32, device=dev),
        "err": torch.zeros(1, dtype=torch.int32, device=dev),
    }
    if all_kv:
        o["all_kv"] = torch.zeros((T, inp.top_k + inp.window, inp.head_dim), dtype=torch.bfloat16,
                                  device=dev)
    if keep:
        o["scores"] = torch.zeros((T, mv), dtype=torch.float32, device=dev)
        o["idx"] = torch.zeros((T, inp.top_k), dtype=torch.int32, device=dev)
        o["count"] = torch.zeros(T, dtype=torch.int32, device=dev)
        o["n_kv"] = torch.zeros(T, dtype=torch.int32, device=dev)
    return o


def run_decode_step(inp, dev, sink: Optional[torch.Tensor] = None, all_kv: bool = True,
                    e4m3: bool = False, one_sequence: bool = False) -> dict:
    """Upload a batch, run one csa_decode_step, return host copies (with
    e4m3, the indexer queries and keys are quantised on the GPU first and
    their codes and scales are returned too)."""
    d = upload(inp, dev)
    if e4m3:
        d = quantize_indexer_e4m3(d)
    outs = alloc_step_outputs(inp, dev, all_kv=all_kv)
    a = step_args(inp, d, outs, sink=sink, e4m3=e4m3, one_sequence=one_sequence)
    ws = step_workspace(a, dev)
    csa_decode_step(a, ws)
    torch.cuda.synchronize(dev)
    res = {k: v.cpu() for k, v in outs.items()}
    r = {
        "scores": res["scores"].numpy(), "idx": res["idx"].numpy(), "count": res["count"].numpy(),
        "n_kv": res["n_kv"].numpy(), "lse": res["lse"].numpy(), "err": int(res["err"][0]),
        "out": res["out"].float().numpy(),
    }
    if all_kv:
        r["all_kv"] = res["all_kv"].view(torch.int16).numpy().view(np.uint16)
    if e4m3:
        for k in ("q_idx8", "q_scale", "k_idx8", "k_scale"):
            r[k] = d[k].cpu().numpy()
    return r
