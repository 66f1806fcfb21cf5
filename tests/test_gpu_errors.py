"""The C-ABI's argument checks on the GPU: every malformed call returns its
documented status (include/dsa.h) with a message from dsa_last_error,
launches nothing and leaves the outputs untouched, and a well-formed call
right after it still matches the oracle's selections."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from gpu_common import log, gpu_arch
from oracle import oracle as O
from deepseek_sparse_attention_amd import binding as B
from deepseek_sparse_attention_amd import inputs as I
from deepseek_sparse_attention_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu


def setup_module():
    assert gpu_arch().startswith("gfx950")


@pytest.fixture(scope="module")
def dw():
    w = I.make_workload("errors", 302, dict(I.GEOM_TOKEN), 2, 5000, [0, 1], [5000, 3001])
    return DeviceWorkload(w)


def _step(dw, geom=None, batch=None, key_stride=None, cache_stride=None, sel_ld=None, ws=None, ws_bytes=None,
          q=None, out=None):
    """dsa_decode_step on dw's tensors with one argument replaced."""
    g = B.geometry(geom or dw.geom)
    ws = dw.ws if ws is None else ws
    ws_ptr = None if ws is False else ctypes.c_void_p(ws.data_ptr() + (1 if ws_bytes == "misaligned" else 0))
    n_ws = 0 if ws is False else (ws.numel() if ws_bytes in (None, "misaligned") else ws_bytes)
    return B._lib.dsa_decode_step(
        ctypes.byref(g), ctypes.byref(batch or dw.batch), B._ptr(dw.idx_q), B._ptr(dw.idx_w), B._ptr(dw.idx_k),
        dw.w.key_rows if key_stride is None else key_stride,
        B._ptr(dw.q) if q is None else q, B._ptr(dw.cache), dw.w.T if cache_stride is None else cache_stride,
        B._ptr(dw.sel), dw.sel_ld if sel_ld is None else sel_ld, B._ptr(dw.sel_count),
        B._ptr(dw.out) if out is None else out, B._ptr(dw.lse), ws_ptr, n_ws, B._stream(None))


def _bad_geoms(g0):
    yield "n_heads", dict(g0, n_heads=32), B.DSA_ERR_UNSUPPORTED
    yield "d_latent", dict(g0, d_latent=256), B.DSA_ERR_UNSUPPORTED
    yield "d_rope", dict(g0, d_rope=32), B.DSA_ERR_UNSUPPORTED
    yield "kpool", dict(g0, kpool=2), B.DSA_ERR_UNSUPPORTED
    yield "top_k 0", dict(g0, top_k=0), B.DSA_ERR_UNSUPPORTED
    yield "top_k big", dict(g0, top_k=4097), B.DSA_ERR_UNSUPPORTED
    yield "top_k % kpool", dict(g0, kpool=4, d_rope=0, top_k=2046), B.DSA_ERR_UNSUPPORTED
    yield "scale 0", dict(g0, softmax_scale=0.0), B.DSA_ERR_UNSUPPORTED
    yield "scale nan", dict(g0, softmax_scale=float("nan")), B.DSA_ERR_UNSUPPORTED
    yield "idx_f16 2", dict(g0, idx_f16=2), B.DSA_ERR_UNSUPPORTED
    yield "f16 pools", dict(g0, kpool=4, d_rope=0, idx_f16=1), B.DSA_ERR_UNSUPPORTED


def test_rejected_calls_leave_outputs_untouched(dw):
    log("C-ABI error paths")
    torch.cuda.synchronize()
    dw.sel.fill_(-7)
    dw.out.fill_(123.0)
    torch.cuda.synchronize()
    cases = [(name, dict(geom=g), want) for name, g, want in _bad_geoms(dw.geom)]
    b = dw.batch
    mk = lambda **kw: B.Batch(kw.get("n_q", b.n_q), kw.get("n_seq", b.n_seq), kw.get("q_seq", b.q_seq),
                              kw.get("q_nvis", b.q_nvis), kw.get("max_nvis", b.max_nvis), b.q_per_seq_hint)
    cases += [
        ("n_q 0", dict(batch=mk(n_q=0)), B.DSA_ERR_ARG),
        ("n_q 65536", dict(batch=mk(n_q=65536)), B.DSA_ERR_UNSUPPORTED),
        ("n_seq 0", dict(batch=mk(n_seq=0)), B.DSA_ERR_ARG),
        ("q_nvis NULL", dict(batch=mk(q_nvis=None)), B.DSA_ERR_ARG),
        ("q_seq NULL, n_q > n_seq", dict(batch=mk(q_seq=None, n_seq=1)), B.DSA_ERR_ARG),
        ("max_nvis 0", dict(batch=mk(max_nvis=0)), B.DSA_ERR_ARG),
        ("max_nvis 2^31", dict(batch=mk(max_nvis=1 << 31)), B.DSA_ERR_ARG),
        ("q_nvis misaligned", dict(batch=mk(q_nvis=b.q_nvis + 4)), B.DSA_ERR_ARG),
        ("key stride", dict(key_stride=dw.max_nvis - 1), B.DSA_ERR_ARG),
        ("cache stride", dict(cache_stride=dw.max_nvis - 1), B.DSA_ERR_ARG),
        ("sel_ld", dict(sel_ld=dw.geom["top_k"] - 1), B.DSA_ERR_ARG),
        ("q NULL", dict(q=ctypes.c_void_p(0)), B.DSA_ERR_ARG),
        ("out misaligned", dict(out=ctypes.c_void_p(dw.out.data_ptr() + 8)), B.DSA_ERR_ARG),
        ("workspace NULL", dict(ws=False), B.DSA_ERR_WORKSPACE),
        ("workspace small", dict(ws_bytes=dw.ws.numel() - 256), B.DSA_ERR_WORKSPACE),
        ("workspace misaligned", dict(ws_bytes="misaligned"), B.DSA_ERR_ARG),
    ]
    for name, kw, want in cases:
        got = _step(dw, **kw)
        msg = B._lib.dsa_last_error().decode()
        assert got == want, f"{name}: status {got}, want {want} ({msg})"
        assert msg, f"{name}: no message"
    torch.cuda.synchronize()
    assert bool((dw.sel == -7).all()) and bool((dw.out == 123.0).all()), "a rejected call wrote its outputs"
    assert B._lib.dsa_workspace_bytes(ctypes.byref(B.geometry(dw.geom)), 65536, 5000) == 0
    assert B._lib.dsa_workspace_bytes(ctypes.byref(B.geometry(dw.geom)), 0, 5000) == 0


def test_good_call_after_rejected_ones(dw):
    """The rejected calls above left no state behind: the next call's
    selections equal the oracle's."""
    log("good call after errors")
    assert _step(dw, sel_ld=dw.geom["top_k"] - 1) == B.DSA_ERR_ARG
    assert _step(dw) == B.DSA_OK
    torch.cuda.synchronize()
    w = dw.w
    scores = O.index_scores(w.q_seq, w.q_nvis, 1, w.idx_q, w.idx_w, w.idx_k)
    sel, cnt = O.topk(w.q_nvis, 1, w.geom["top_k"], scores)
    assert np.array_equal(dw.sel_count.cpu().numpy(), cnt)
    assert np.array_equal(dw.sel.cpu().numpy(), sel)


def _entry_calls(dw, scores, score_ld):
    """(name, thunk) for each entry point of the path on dw's tensors."""
    g, b = dw.geom, dw.batch
    return [
        ("dsa_index_scores", lambda: B.index_scores(g, b, dw.idx_q, dw.idx_w, dw.idx_k, dw.w.key_rows, scores,
                                                     score_ld)),
        ("dsa_topk", lambda: B.topk(g, b, scores, score_ld, dw.sel, dw.sel_ld, dw.sel_count, dw.ws)),
        ("dsa_mla_attend", lambda: B.mla_attend(g, b, dw.q, dw.cache, dw.w.T, dw.sel, dw.sel_ld, dw.sel_count,
                                                 dw.out, dw.lse, dw.ws)),
        ("dsa_decode_step", lambda: dw.decode_step()),
        ("dsa_workspace_init", lambda: B._check(B._lib.dsa_workspace_init(B._ptr(dw.ws), dw.ws.numel(),
                                                                          B._stream(None)), "init")),
    ]


def test_injected_launch_failure_is_reported(dw, monkeypatch):
    """DSA_TEST_FAIL_LAUNCH=1 makes every entry point take its launch-failure
    path after its argument checks: DSA_ERR_LAUNCH with a message, nothing
    written.  Unset, the same calls run and the step matches the oracle."""
    log("injected launch failures")
    score_ld = dw.max_nvis
    scores = torch.full((dw.n_q, score_ld), 5.0, device="cuda")
    torch.cuda.synchronize()
    dw.sel.fill_(-7)
    monkeypatch.setenv("DSA_TEST_FAIL_LAUNCH", "1")
    for name, call in _entry_calls(dw, scores, score_ld):
        with pytest.raises(B.DSAError) as e:
            call()
        assert e.value.status == B.DSA_ERR_LAUNCH, f"{name}: {e.value}"
        assert "injected" in str(e.value), f"{name}: {e.value}"
    torch.cuda.synchronize()
    assert bool((scores == 5.0).all()) and bool((dw.sel == -7).all()), "a failed launch wrote its outputs"
    monkeypatch.delenv("DSA_TEST_FAIL_LAUNCH")
    for name, call in _entry_calls(dw, scores, score_ld):
        call()
    torch.cuda.synchronize()
    test_good_call_after_rejected_ones(dw)


def test_split_entry_points_check_their_own_arguments(dw):
    """dsa_index_scores, dsa_topk and dsa_mla_attend refuse short row
    strides, NULL outputs and a short workspace with their documented
    statuses."""
    log("split entry point checks")
    g, b = B.geometry(dw.geom), dw.batch
    score_ld = dw.max_nvis
    scores = torch.zeros((dw.n_q, score_ld), device="cuda")
    P, s = B._ptr, B._stream(None)
    ws, n_ws = P(dw.ws), dw.ws.numel()
    L = B._lib
    cases = [
        ("scores: key stride", L.dsa_index_scores(ctypes.byref(g), ctypes.byref(b), P(dw.idx_q), P(dw.idx_w),
                                                  P(dw.idx_k), dw.max_nvis - 1, P(scores), score_ld, s),
         B.DSA_ERR_ARG),
        ("scores: score_ld", L.dsa_index_scores(ctypes.byref(g), ctypes.byref(b), P(dw.idx_q), P(dw.idx_w),
                                                P(dw.idx_k), dw.w.key_rows, P(scores), dw.max_nvis - 1, s),
         B.DSA_ERR_ARG),
        ("scores: NULL scores", L.dsa_index_scores(ctypes.byref(g), ctypes.byref(b), P(dw.idx_q), P(dw.idx_w),
                                                   P(dw.idx_k), dw.w.key_rows, None, score_ld, s), B.DSA_ERR_ARG),
        ("topk: score_ld", L.dsa_topk(ctypes.byref(g), ctypes.byref(b), P(scores), dw.max_nvis - 1, P(dw.sel),
                                      dw.sel_ld, P(dw.sel_count), ws, n_ws, s), B.DSA_ERR_ARG),
        ("topk: sel_ld", L.dsa_topk(ctypes.byref(g), ctypes.byref(b), P(scores), score_ld, P(dw.sel),
                                    dw.sel_ld - 1, P(dw.sel_count), ws, n_ws, s), B.DSA_ERR_ARG),
        ("topk: NULL count", L.dsa_topk(ctypes.byref(g), ctypes.byref(b), P(scores), score_ld, P(dw.sel),
                                        dw.sel_ld, None, ws, n_ws, s), B.DSA_ERR_ARG),
        ("topk: short workspace", L.dsa_topk(ctypes.byref(g), ctypes.byref(b), P(scores), score_ld, P(dw.sel),
                                             dw.sel_ld, P(dw.sel_count), ws, 256, s), B.DSA_ERR_WORKSPACE),
        ("attend: cache stride", L.dsa_mla_attend(ctypes.byref(g), ctypes.byref(b), P(dw.q), P(dw.cache),
                                                  dw.max_nvis - 1, P(dw.sel), dw.sel_ld, P(dw.sel_count),
                                                  P(dw.out), P(dw.lse), ws, n_ws, s), B.DSA_ERR_ARG),
        ("attend: NULL sel", L.dsa_mla_attend(ctypes.byref(g), ctypes.byref(b), P(dw.q), P(dw.cache), dw.w.T,
                                              None, dw.sel_ld, P(dw.sel_count), P(dw.out), P(dw.lse), ws, n_ws, s),
         B.DSA_ERR_ARG),
        ("attend: no workspace", L.dsa_mla_attend(ctypes.byref(g), ctypes.byref(b), P(dw.q), P(dw.cache), dw.w.T,
                                                  P(dw.sel), dw.sel_ld, P(dw.sel_count), P(dw.out), P(dw.lse), None,
                                                  0, s), B.DSA_ERR_WORKSPACE),
    ]
    for name, got, want in cases:
        assert got == want, f"{name}: status {got}, want {want} ({B._lib.dsa_last_error().decode()})"
