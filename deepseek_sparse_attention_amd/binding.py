"""Thin ctypes binding of ``libdsa.so`` (the C ABI in ``include/dsa.h``).

Argument marshalling only: torch supplies device memory and the current
stream, every step runs in the HIP kernels behind the C ABI.  There is no
fallback: if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_OK, DSA_ERR_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_DEVICE, DSA_ERR_LAUNCH = 0, -1, -2, -3, -4, -5


class Geometry(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("n_idx_heads", ctypes.c_int32), ("d_idx", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("kpool", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("idx_f16", ctypes.c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_seq", ctypes.c_int32), ("q_seq", ctypes.c_void_p),
                ("q_nvis", ctypes.c_void_p), ("max_nvis", ctypes.c_int64), ("q_per_seq_hint", ctypes.c_int32)]


EXPORTS = ("dsa_workspace_bytes", "dsa_workspace_init", "dsa_index_scores", "dsa_topk", "dsa_mla_attend",
           "dsa_decode_step", "dsa_pool_append", "dsa_absorb_query", "dsa_project_output", "dsa_index_prepare",
           "dsa_status_str", "dsa_last_error", "dsa_device_check", "dsa_set_timing_events", "dsa_timing_ran",
           "dsa_stream_read", "dsa_decode_step_noalloc")


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m deepseek_sparse_attention_amd.build`")
    L = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    G, B = ctypes.POINTER(Geometry), ctypes.POINTER(Batch)
    sig = {
        "dsa_workspace_bytes": (sz, [G, i32, i64]),
        "dsa_workspace_init": (ctypes.c_int, [P, sz, P]),
        "dsa_index_scores": (ctypes.c_int, [G, B, P, P, P, i64, P, i64, P]),
        "dsa_topk": (ctypes.c_int, [G, B, P, i64, P, i32, P, P, sz, P]),
        "dsa_mla_attend": (ctypes.c_int, [G, B, P, P, i64, P, i32, P, P, P, P, sz, P]),
        "dsa_decode_step": (ctypes.c_int, [G, B, P, P, P, i64, P, P, i64, P, i32, P, P, P, P, sz, P]),
        "dsa_decode_step_noalloc": (ctypes.c_int, [G, B, P, P, P, i64, P, P, i64, P, i32, P, P, P, P]),
        "dsa_pool_append": (ctypes.c_int, [i32, P, P, i32, P, i64, P, P, i64, P, P]),
        "dsa_absorb_query": (ctypes.c_int, [i32, i32, P, P, P, P, P]),
        "dsa_project_output": (ctypes.c_int, [i32, P, P, P, P]),
        "dsa_index_prepare": (ctypes.c_int, [G, B, ctypes.c_double, P, P, i32, P, P, P, P, i64, P]),
        "dsa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "dsa_last_error": (ctypes.c_char_p, []),
        "dsa_device_check": (ctypes.c_int, []),
        "dsa_set_timing_events": (ctypes.c_int, [P, i32]),
        "dsa_timing_ran": (i32, []),
        "dsa_stream_read": (ctypes.c_int, [P, sz, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


_lib = load_library()


class DSAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = _lib.dsa_last_error().decode()
        super().__init__(f"{what}: {_lib.dsa_status_str(status).decode()} ({status}): {detail}")


def _check(status: int, what: str) -> None:
    if status != DSA_OK:
        raise DSAError(status, what)


def geometry(geom: dict) -> Geometry:
    return Geometry(geom["n_heads"], geom["d_latent"], geom["d_rope"], geom["n_idx_heads"], geom["d_idx"],
                    geom["top_k"], geom["kpool"], float(geom["softmax_scale"]), int(geom.get("idx_f16", 0)))


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def batch(q_seq: torch.Tensor | None, q_nvis: torch.Tensor, max_nvis: int, n_seq: int,
          q_per_seq_hint: int = 0) -> Batch:
    """The C struct holds raw device pointers; the returned object keeps the
    two tensors alive for as long as it lives."""
    for t in (q_seq, q_nvis):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError("q_seq / q_nvis must be contiguous int32 device tensors")
    b = Batch(int(q_nvis.shape[0]), int(n_seq), _ptr(q_seq), _ptr(q_nvis), int(max_nvis), int(q_per_seq_hint))
    b._keep = (q_seq, q_nvis)
    return b


def workspace_bytes(geom: dict, n_q: int, max_nvis: int) -> int:
    return int(_lib.dsa_workspace_bytes(ctypes.byref(geometry(geom)), n_q, max_nvis))


def new_workspace(geom: dict, n_q: int, max_nvis: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (uint8) of the size the library asks for."""
    n = workspace_bytes(geom, n_q, max_nvis)
    if n == 0:
        raise DSAError(DSA_ERR_UNSUPPORTED, "workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check(_lib.dsa_workspace_init(_ptr(ws), n, _stream(None)), "dsa_workspace_init")
    return ws


def device_check() -> None:
    _check(_lib.dsa_device_check(), "dsa_device_check")


def index_scores(geom: dict, b: Batch, idx_q, idx_w, idx_k, key_seq_stride: int, scores, score_ld: int,
                 stream=None) -> None:
    _check(_lib.dsa_index_scores(ctypes.byref(geometry(geom)), ctypes.byref(b), _ptr(idx_q), _ptr(idx_w),
                                 _ptr(idx_k), int(key_seq_stride), _ptr(scores), int(score_ld), _stream(stream)),
           "dsa_index_scores")


def topk(geom: dict, b: Batch, scores, score_ld: int, sel, sel_ld: int, sel_count, ws, stream=None) -> None:
    _check(_lib.dsa_topk(ctypes.byref(geometry(geom)), ctypes.byref(b), _ptr(scores), int(score_ld), _ptr(sel),
                         int(sel_ld), _ptr(sel_count), _ptr(ws), ws.numel() if ws is not None else 0,
                         _stream(stream)), "dsa_topk")


def mla_attend(geom: dict, b: Batch, q, cache, cache_seq_stride: int, sel, sel_ld: int, sel_count, out, lse, ws,
               stream=None) -> None:
    _check(_lib.dsa_mla_attend(ctypes.byref(geometry(geom)), ctypes.byref(b), _ptr(q), _ptr(cache),
                               int(cache_seq_stride), _ptr(sel), int(sel_ld), _ptr(sel_count), _ptr(out), _ptr(lse),
                               _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)), "dsa_mla_attend")


def decode_step(geom: dict, b: Batch, idx_q, idx_w, idx_k, key_seq_stride: int, q, cache, cache_seq_stride: int,
                sel, sel_ld: int, sel_count, out, lse, ws, stream=None) -> None:
    _check(_lib.dsa_decode_step(ctypes.byref(geometry(geom)), ctypes.byref(b), _ptr(idx_q), _ptr(idx_w),
                                _ptr(idx_k), int(key_seq_stride), _ptr(q), _ptr(cache), int(cache_seq_stride),
                                _ptr(sel), int(sel_ld), _ptr(sel_count), _ptr(out), _ptr(lse), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(stream)), "dsa_decode_step")


def decode_step_noalloc(geom: dict, b: Batch, idx_q, idx_w, idx_k, key_seq_stride: int, q, cache,
                        cache_seq_stride: int, sel, sel_ld: int, sel_count, out, lse, stream=None) -> None:
    """The fused step on the library's own device scratch (no workspace)."""
    _check(_lib.dsa_decode_step_noalloc(ctypes.byref(geometry(geom)), ctypes.byref(b), _ptr(idx_q), _ptr(idx_w),
                                        _ptr(idx_k), int(key_seq_stride), _ptr(q), _ptr(cache),
                                        int(cache_seq_stride), _ptr(sel), int(sel_ld), _ptr(sel_count), _ptr(out),
                                        _ptr(lse), _stream(stream)), "dsa_decode_step_noalloc")


def pool_append(n_tok, n_new, max_new: int, new_kg, rolling, pool_keys, pos_emb, stream=None) -> None:
    """k-pool key producer.  n_tok, n_new: int32 [n_seq]; new_kg: bf16 bits
    (int16/uint16) [n_seq, new_stride, 256]; rolling [n_seq, 4, 256];
    pool_keys [n_seq, pool_stride, 128]; pos_emb float32 [4, 128]; all cuda."""
    for t, dt in ((n_tok, torch.int32), (n_new, torch.int32), (pos_emb, torch.float32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"expected a contiguous cuda {dt} tensor, got {t.dtype} on {t.device}")
    for t in (new_kg, rolling, pool_keys):
        if t.element_size() != 2 or not t.is_cuda or not t.is_contiguous():
            raise TypeError("cells, rolling buffer and pool keys are contiguous 16-bit cuda tensors")
    n_seq = int(n_tok.shape[0])
    if new_kg.shape[0] != n_seq or rolling.shape != (n_seq, 4, 256) or pool_keys.shape[0] != n_seq:
        raise ValueError("shapes: new_kg [n_seq, stride, 256], rolling [n_seq, 4, 256], pool_keys [n_seq, P, 128]")
    _check(_lib.dsa_pool_append(n_seq, _ptr(n_tok), _ptr(n_new), int(max_new), _ptr(new_kg), int(new_kg.shape[1]),
                                _ptr(rolling), _ptr(pool_keys), int(pool_keys.shape[1]), _ptr(pos_emb),
                                _stream(stream)), "dsa_pool_append")


def absorb_query(q_nope, q_rope, w_uk, q_abs, stream=None) -> None:
    """q_nope [n_q, 64, 256], q_rope [n_q, 64, d_rope] or None, w_uk [64, 256, 512],
    q_abs [n_q, 64, 512 + d_rope]: 16-bit (bf16 bits) contiguous cuda tensors."""
    for t in (q_nope, w_uk, q_abs) + ((q_rope,) if q_rope is not None else ()):
        if t.element_size() != 2 or not t.is_cuda or not t.is_contiguous():
            raise TypeError("absorb_query takes contiguous 16-bit cuda tensors")
    n_q = int(q_nope.shape[0])
    d_rope = 0 if q_rope is None else int(q_rope.shape[2])
    if tuple(q_nope.shape) != (n_q, 64, 256) or tuple(w_uk.shape) != (64, 256, 512) or \
            tuple(q_abs.shape) != (n_q, 64, 512 + d_rope):
        raise ValueError("shapes: q_nope [n_q, 64, 256], w_uk [64, 256, 512], q_abs [n_q, 64, 512 + d_rope]")
    _check(_lib.dsa_absorb_query(n_q, d_rope, _ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(q_abs), _stream(stream)),
           "dsa_absorb_query")


def project_output(o, w_uv, ctx, stream=None) -> None:
    """o float32 [n_q, 64, 512], w_uv 16-bit [64, 256, 512], ctx float32 [n_q, 64, 256]."""
    n_q = int(o.shape[0])
    if o.dtype != torch.float32 or ctx.dtype != torch.float32 or w_uv.element_size() != 2:
        raise TypeError("project_output: o and ctx float32, w_uv 16-bit")
    if tuple(o.shape) != (n_q, 64, 512) or tuple(w_uv.shape) != (64, 256, 512) or tuple(ctx.shape) != (n_q, 64, 256):
        raise ValueError("shapes: o [n_q, 64, 512], w_uv [64, 256, 512], ctx [n_q, 64, 256]")
    for t in (o, w_uv, ctx):
        if not t.is_cuda or not t.is_contiguous():
            raise TypeError("project_output takes contiguous cuda tensors")
    _check(_lib.dsa_project_output(n_q, _ptr(o), _ptr(w_uv), _ptr(ctx), _stream(stream)), "dsa_project_output")


def index_prepare(geom: dict, b: Batch, q_in, q_out, k_seq, k_pos, k_in, idx_k, key_seq_stride: int,
                  rope_base: float = 8.0e6, stream=None) -> None:
    """Rope + Hadamard rotation + 16-bit rounding of indexer queries (q_in
    float32 [n_q, 32, 128] -> q_out 16-bit, or both None) and of new keys
    (k_in float32 [n_new, 128] at k_pos int32 [n_new] of k_seq int32 [n_new]
    or None, written into idx_k 16-bit [n_seq, key_seq_stride, 128]).  The
    16-bit format is the geometry's idx_f16."""
    n_new = 0 if k_pos is None else int(k_pos.shape[0])
    if q_in is not None and q_out is not None:     # one without the other is refused by the library
        if q_in.dtype != torch.float32 or q_out.element_size() != 2 or tuple(q_in.shape) != tuple(q_out.shape):
            raise TypeError("index_prepare: q_in float32 and q_out 16-bit of one shape")
    if n_new:
        if k_in.dtype != torch.float32 or tuple(k_in.shape) != (n_new, 128) or idx_k.element_size() != 2:
            raise TypeError("index_prepare: k_in float32 [n_new, 128], idx_k 16-bit")
        if k_pos.dtype != torch.int32 or (k_seq is not None and k_seq.dtype != torch.int32):
            raise TypeError("index_prepare: k_pos and k_seq int32")
    for t in (q_in, q_out, k_seq, k_pos, k_in, idx_k):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise TypeError("index_prepare takes contiguous cuda tensors")
    _check(_lib.dsa_index_prepare(ctypes.byref(geometry(geom)), ctypes.byref(b), float(rope_base), _ptr(q_in),
                                  _ptr(q_out), n_new, _ptr(k_seq), _ptr(k_pos), _ptr(k_in), _ptr(idx_k),
                                  int(key_seq_stride), _stream(stream)), "dsa_index_prepare")


def stream_read(buf, sink, stream=None) -> None:
    """Bandwidth probe: reads all of buf (a contiguous cuda tensor whose byte
    size is a multiple of 16) with streaming loads; sink: an int32 cuda
    tensor of at least one element."""
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda or sink.dtype != torch.int32:
        raise TypeError("buf: a contiguous cuda tensor; sink: an int32 cuda tensor")
    _check(_lib.dsa_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)),
           "dsa_stream_read")


def timing_ran() -> int:
    """Bit i set: the last dsa_decode_step on this thread ran kernel i
    (score, filter, select, attend, merge)."""
    return int(_lib.dsa_timing_ran())


def set_timing_events(events) -> None:
    """events: a list of torch.cuda.Event(enable_timing=True), or None to stop.
    dsa_decode_step launches its i-th kernel with events[2i] and
    events[2i + 1] as that kernel's own start and stop marks."""
    if not events:
        _lib.dsa_set_timing_events(None, 0)
        set_timing_events._keep = None
        return
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    set_timing_events._keep = (arr, events)
    _check(_lib.dsa_set_timing_events(ctypes.cast(arr, ctypes.c_void_p), len(events)), "dsa_set_timing_events")
