"""ctypes front of the C oracle (``dsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path may
not.  It imports nothing from the HIP package.  All arrays are numpy, bf16
tensors are passed as their raw uint16 bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dsa_oracle.c")
LIB = os.path.join(HERE, "libdsa_oracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP over queries / rows)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp",
                               "-fPIC", "-shared", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def load(path: str):
    """Load an oracle shared library and declare its C signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    f64 = ctypes.c_double
    L.oracle_index_scores.argtypes = [i32, P, P, i32, i32, i32, P, P, P, i64, P, i64, i32]
    L.oracle_topk.argtypes = [i32, P, i32, i32, P, i64, P, i32, P]
    L.oracle_mla_attend.argtypes = [i32, P, i32, i32, i32, f32, P, P, i64, P, i32, P, P, P]
    L.oracle_decode_step.argtypes = [i32, P, P, i32, i32, i32, i32, i32, f32, i32, i32,
                                     P, P, P, i64, P, P, i64, P, i32, P, P, P, i32]
    L.oracle_max_threads.argtypes = []
    L.oracle_set_threads.argtypes = [i32]
    L.oracle_set_threads.restype = None
    L.oracle_pool_append.argtypes = [i32, P, P, P, i64, i32, P, P, i64, P]
    L.oracle_absorb_query.argtypes = [i32, i32, i32, i32, i32, P, P, P, P]
    L.oracle_project_output.argtypes = [i32, i32, i32, i32, P, P, P]
    L.oracle_index_rotate.argtypes = [i32, i32, f64, i64, P, P]
    L.oracle_index_rotate.restype = None
    L.oracle_round16.argtypes = [i64, P, P, i32]
    L.oracle_round16.restype = None
    L.oracle_index_prepare.argtypes = [i32, i32, i32, i32, f64, P, P, P, i32, i32, P, P, P, P, i64, i32]
    for f in (L.oracle_index_scores, L.oracle_topk, L.oracle_mla_attend,
              L.oracle_decode_step, L.oracle_max_threads):
        f.restype = ctypes.c_int
    return L


_default = None


def lib():
    global _default
    if _default is None:
        _default = load(build())
    return _default


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads(L=None) -> int:
    return int((L or lib()).oracle_max_threads())


def set_threads(n: int, L=None) -> None:
    """Thread count of the oracle's OpenMP loops from now on (timing only)."""
    (L or lib()).oracle_set_threads(int(n))


def index_scores(q_seq, q_nvis, kpool, idx_q, idx_w, idx_k, score_ld=None, fill=np.nan, L=None,
                 f16=False):
    """Scores [n_q, score_ld] float32; entries past rows(q) hold ``fill``.

    idx_q: uint16 [n_q, HI, DI]; idx_w: float32 [n_q, HI];
    idx_k: uint16 [n_seq, key_rows, DI]; 16-bit elements are bf16, or IEEE
    f16 when ``f16``."""
    q_seq, q_nvis = _c(q_seq, np.int32), _c(q_nvis, np.int32)
    idx_q, idx_w, idx_k = _c(idx_q, np.uint16), _c(idx_w, np.float32), _c(idx_k, np.uint16)
    n_q, HI, DI = idx_q.shape
    if score_ld is None:
        score_ld = max(1, int(q_nvis.max()) // kpool)
    out = np.full((n_q, score_ld), fill, dtype=np.float32)
    rc = (L or lib()).oracle_index_scores(n_q, _p(q_seq), _p(q_nvis), kpool, HI, DI, _p(idx_q),
                                   _p(idx_w), _p(idx_k), idx_k.shape[1], _p(out), score_ld, int(f16))
    assert rc == 0
    return out


def topk(q_nvis, kpool, top_k, scores, sel_ld=None, L=None):
    """Returns (sel int32 [n_q, sel_ld] ascending, padded -1; count int32 [n_q])."""
    q_nvis = _c(q_nvis, np.int32)
    scores = _c(scores, np.float32)
    n_q = q_nvis.shape[0]
    if sel_ld is None:
        sel_ld = top_k + kpool - 1
    sel = np.empty((n_q, sel_ld), dtype=np.int32)
    cnt = np.empty(n_q, dtype=np.int32)
    rc = (L or lib()).oracle_topk(n_q, _p(q_nvis), kpool, top_k, _p(scores), scores.shape[1],
                           _p(sel), sel_ld, _p(cnt))
    if rc != 0:
        raise ValueError("sel_ld too small for the selection")
    return sel, cnt


def mla_attend(q_seq, d_latent, d_rope, scale, q, cache, sel, sel_count, want_lse=True, L=None):
    """Returns (out float32 [n_q, H, d_latent], lse float32 [n_q, H] or None).

    q: uint16 [n_q, H, D]; cache: uint16 [n_seq, T, D]."""
    q_seq = _c(q_seq, np.int32)
    q, cache = _c(q, np.uint16), _c(cache, np.uint16)
    sel, sel_count = _c(sel, np.int32), _c(sel_count, np.int32)
    n_q, H, D = q.shape
    assert D == d_latent + d_rope and cache.shape[2] == D
    out = np.empty((n_q, H, d_latent), dtype=np.float32)
    lse = np.empty((n_q, H), dtype=np.float32) if want_lse else None
    rc = (L or lib()).oracle_mla_attend(n_q, _p(q_seq), H, d_latent, d_rope, float(scale), _p(q),
                                 _p(cache), cache.shape[1], _p(sel), sel.shape[1],
                                 _p(sel_count), _p(out), _p(lse))
    assert rc == 0
    return out, lse


def decode_step(geom, q_seq, q_nvis, idx_q, idx_w, idx_k, q, cache, sel_ld=None, L=None):
    """Full step for every query.  Returns (sel, sel_count, out, lse).  The
    indexer elements are f16 when ``geom.get("idx_f16")``, else bf16."""
    q_seq, q_nvis = _c(q_seq, np.int32), _c(q_nvis, np.int32)
    idx_q, idx_w, idx_k = _c(idx_q, np.uint16), _c(idx_w, np.float32), _c(idx_k, np.uint16)
    q, cache = _c(q, np.uint16), _c(cache, np.uint16)
    kpool, top_k = geom["kpool"], geom["top_k"]
    n_q, H, D = q.shape
    if sel_ld is None:
        sel_ld = top_k + kpool - 1
    sel = np.empty((n_q, sel_ld), dtype=np.int32)
    cnt = np.empty(n_q, dtype=np.int32)
    out = np.empty((n_q, H, geom["d_latent"]), dtype=np.float32)
    lse = np.empty((n_q, H), dtype=np.float32)
    rc = (L or lib()).oracle_decode_step(n_q, _p(q_seq), _p(q_nvis), kpool, top_k, H,
                                  geom["d_latent"], geom["d_rope"], float(geom["softmax_scale"]),
                                  idx_q.shape[1], idx_q.shape[2], _p(idx_q), _p(idx_w),
                                  _p(idx_k), idx_k.shape[1], _p(q), _p(cache), cache.shape[1],
                                  _p(sel), sel_ld, _p(cnt), _p(out), _p(lse),
                                  int(geom.get("idx_f16", 0)))
    assert rc == 0
    return sel, cnt, out, lse


def pool_append(n_tok, n_new, new_kg, rolling, pool_keys, pos_emb, L=None):
    """k-pool key producer, token by token.  Updates ``rolling`` and
    ``pool_keys`` in place (uint16 bf16 bits) and returns them.

    n_tok, n_new: int [n_seq]; new_kg: uint16 [n_seq, new_stride, 2 d_idx];
    rolling: uint16 [n_seq, 4, 2 d_idx]; pool_keys: uint16 [n_seq, pool_stride, d_idx];
    pos_emb: float32 [4, d_idx]."""
    n_tok, n_new = _c(n_tok, np.int32), _c(n_new, np.int32)
    new_kg, pos_emb = _c(new_kg, np.uint16), _c(pos_emb, np.float32)
    assert rolling.dtype == np.uint16 and rolling.flags.c_contiguous
    assert pool_keys.dtype == np.uint16 and pool_keys.flags.c_contiguous
    n_seq, stride, cell = new_kg.shape
    d_idx = cell // 2
    assert rolling.shape == (n_seq, 4, cell) and pool_keys.shape[0] == n_seq and pool_keys.shape[2] == d_idx
    assert pos_emb.shape == (4, d_idx) and (n_new <= stride).all()
    assert ((n_tok + n_new) // 4 <= pool_keys.shape[1]).all()
    rc = (L or lib()).oracle_pool_append(n_seq, _p(n_tok), _p(n_new), _p(new_kg), stride, d_idx,
                                         _p(rolling), _p(pool_keys), pool_keys.shape[1], _p(pos_emb))
    assert rc == 0
    return rolling, pool_keys


def absorb_query(q_nope, q_rope, w_uk, L=None):
    """q_abs (uint16 bf16 [n_q, H, d_latent + d_rope]) from q_nope [n_q, H, d_nope],
    q_rope [n_q, H, d_rope] (or None for d_rope 0) and w_uk [H, d_nope, d_latent]."""
    q_nope, w_uk = _c(q_nope, np.uint16), _c(w_uk, np.uint16)
    n_q, H, dn = q_nope.shape
    assert w_uk.shape[:2] == (H, dn)
    dl = w_uk.shape[2]
    if q_rope is None:
        q_rope = np.zeros((n_q, H, 0), np.uint16)
    q_rope = _c(q_rope, np.uint16)
    dr = q_rope.shape[2]
    out = np.empty((n_q, H, dl + dr), np.uint16)
    rc = (L or lib()).oracle_absorb_query(n_q, H, dn, dl, dr, _p(q_nope), _p(q_rope), _p(w_uk), _p(out))
    assert rc == 0
    return out


def project_output(o, w_uv, L=None):
    """ctx (float32 [n_q, H, d_v]) from o float32 [n_q, H, d_latent] and w_uv [H, d_v, d_latent]."""
    o, w_uv = _c(o, np.float32), _c(w_uv, np.uint16)
    n_q, H, dl = o.shape
    assert w_uv.shape[0] == H and w_uv.shape[2] == dl
    dv = w_uv.shape[1]
    out = np.empty((n_q, H, dv), np.float32)
    rc = (L or lib()).oracle_project_output(n_q, H, dl, dv, _p(o), _p(w_uv), _p(out))
    assert rc == 0
    return out


ROPE_BASE = 8.0e6


def index_rotate(x, pos, d_rope, base=ROPE_BASE, L=None):
    """Rope then orthonormal Walsh-Hadamard rotation of one vector, in double
    and unrounded.  x: float64 [d_idx]."""
    x = _c(x, np.float64)
    y = np.empty_like(x)
    (L or lib()).oracle_index_rotate(x.shape[0], int(d_rope), float(base), int(pos), _p(x), _p(y))
    return y


def round16(v, f16, L=None):
    """Nearest bf16 (or IEEE f16) bits of float64 values, ties to even."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    (L or lib()).oracle_round16(v.size, _p(v), _p(out), int(f16))
    return out


def index_prepare(q_nvis, q_in, k_seq, k_pos, k_in, k_cache, d_rope, f16, base=ROPE_BASE, L=None):
    """Indexer queries (returned, uint16 [n_q, HI, DI]) and keys (appended in
    place to ``k_cache`` uint16 [n_seq, stride, DI], which is returned too).

    q_nvis int [n_q]; q_in float32 [n_q, HI, DI]; k_seq int [n_new] or None;
    k_pos int [n_new]; k_in float32 [n_new, DI]."""
    q_nvis, q_in = _c(q_nvis, np.int32), _c(q_in, np.float32)
    k_pos, k_in = _c(k_pos, np.int32), _c(k_in, np.float32)
    k_seq = None if k_seq is None else _c(k_seq, np.int32)
    assert k_cache.dtype == np.uint16 and k_cache.flags.c_contiguous
    n_q, HI, DI = q_in.shape
    n_new = k_pos.shape[0]
    assert k_in.shape == (n_new, DI) and k_cache.shape[2] == DI
    q_out = np.empty((n_q, HI, DI), np.uint16)
    rc = (L or lib()).oracle_index_prepare(n_q, HI, DI, int(d_rope), float(base), _p(q_nvis), _p(q_in),
                                           _p(q_out), n_new, k_cache.shape[0], _p(k_seq), _p(k_pos),
                                           _p(k_in), _p(k_cache), k_cache.shape[1], int(f16))
    assert rc == 0
    return q_out, k_cache
