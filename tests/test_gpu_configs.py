"""The five problem configurations and the 128K decode point at full size,
in the launch configuration the benchmark times (the fused step).  The
oracle checks every query of every configuration, including all 512
positions of the prefill chunk (C3)."""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

from gpu_common import check_attention, check_selection, log, oracle_decode

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

from deepseek_sparse_attention_amd import inputs as I             # noqa: E402
from deepseek_sparse_attention_amd.workload import DeviceWorkload  # noqa: E402


def _run(name, queries=None):
    t0 = time.time()
    w = I.config(name)
    log(f"{name}: generated in {time.time() - t0:.1f}s (n_q={w.n_q}, T={w.T})")
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel_g, cnt_g = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    out_g, lse_g = dw.out.cpu().numpy(), dw.lse.cpu().numpy()
    del dw
    torch.cuda.empty_cache()
    t0 = time.time()
    sel, cnt, out, lse = oracle_decode(w, queries)
    log(f"{name}: oracle in {time.time() - t0:.1f}s")
    idx = np.arange(w.n_q) if queries is None else np.asarray(queries)
    check_selection(sel_g[idx], cnt_g[idx], sel, cnt, name)
    check_attention(out_g[idx], lse_g[idx], out, lse, name)
    return w, sel_g, cnt_g


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c4", "m128k"])
def test_config_full(name):
    _run(name)


def test_config_c3_full():
    """Every one of the 512 prefill positions against the oracle (about 20 s
    of oracle time on 16 host threads)."""
    w, sel_g, cnt_g = _run("c3")
    for j in range(w.n_q):
        s = sel_g[j, :cnt_g[j]]
        assert cnt_g[j] == 2048 and np.all(np.diff(s) > 0) and s[-1] < w.q_nvis[j]


@pytest.mark.parametrize("batch", [3, 5, 6])
def test_decode_128k_batch_shapes(batch):
    """Batches at 128K whose launch shapes differ from the 8-query point:
    3 queries score 2,048-row tiles with 8-wave work-groups, 5 and 6
    4,096-row tiles; their attention takes 16, 11 and 8 splits (at most 64
    (query, split) pairs).  Every query against the oracle."""
    t0 = time.time()
    w = I.decode_128k(batch)
    log(f"128K x {batch}: generated in {time.time() - t0:.1f}s")
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel_g, cnt_g = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    out_g, lse_g = dw.out.cpu().numpy(), dw.lse.cpu().numpy()
    del dw
    torch.cuda.empty_cache()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(sel_g, cnt_g, sel, cnt, f"128K x {batch}")
    check_attention(out_g, lse_g, out, lse, f"128K x {batch}")


@pytest.mark.parametrize("n_q", [9, 16, 64, 128])
def test_decode_large_batches(n_q):
    """Decode batches beyond the 8-query point, at 131,072 cached tokens:
    the top-k leaves the attention kernel (k_select), the attention is
    k_attend_wv with the splits widened to at most 64 (query, split) pairs
    up to 64 queries and k_attend with 2 splits at 128.  Queries are dealt
    over 8 sequences in turn (no two neighbours share one, so the batch is
    a decode batch, not a prefill run) and each sees its own context
    length.  Every query against the oracle."""
    T = 131072
    q_seq = np.arange(n_q) % 8
    q_nvis = T - 97 * np.arange(n_q)
    w = I.make_workload(f"large_{n_q}", 60 + n_q % 7, I.GEOM_TOKEN, 8, T, q_seq, q_nvis)
    log(f"decode x {n_q}: workload ready")
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel_g, cnt_g = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    out_g, lse_g = dw.out.cpu().numpy(), dw.lse.cpu().numpy()
    del dw
    torch.cuda.empty_cache()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(sel_g, cnt_g, sel, cnt, f"decode x {n_q}")
    check_attention(out_g, lse_g, out, lse, f"decode x {n_q}")


@pytest.mark.parametrize("window", [2, 5, 9])
def test_verify_windows_full(window):
    """Speculative verify windows at 131,072 cached tokens, 8 sequences of
    `window` rows at their last positions (the prefill scorer with the
    run-length hint, then the per-row chain): every row against the
    oracle."""
    w = I.decode_window(8, window)
    log(f"verify windows 8 x {window} at 131072: workload ready")
    dw = DeviceWorkload(w)
    assert dw.batch.q_per_seq_hint == window
    dw.decode_step()
    torch.cuda.synchronize()
    sel_g, cnt_g = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    out_g, lse_g = dw.out.cpu().numpy(), dw.lse.cpu().numpy()
    del dw
    torch.cuda.empty_cache()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(sel_g, cnt_g, sel, cnt, f"windows 8 x {window}")
    check_attention(out_g, lse_g, out, lse, f"windows 8 x {window}")


def test_kpool_batch_full():
    """The k-pool variant (NoPE, pools of 4) for a batch: 4 sequences of
    2^19 cached tokens whose queries see 2^19 - 1, 2^19 - 2, 2^19 - 3 and
    2^19 - 4 tokens (pool tails of 3, 2, 1 and 0 tokens), so that the
    attention splits and the tail split differ from the one-query C4 case.
    Every query against the oracle."""
    T = 1 << 19
    w = I.make_workload("kpool_b4", 71, I.GEOM_KPOOL, 4, T, np.arange(4), [T - 1, T - 2, T - 3, T - 4])
    log("k-pool x 4 at 2^19: workload ready")
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel_g, cnt_g = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    out_g, lse_g = dw.out.cpu().numpy(), dw.lse.cpu().numpy()
    del dw
    torch.cuda.empty_cache()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(sel_g, cnt_g, sel, cnt, "k-pool x 4")
    check_attention(out_g, lse_g, out, lse, "k-pool x 4")


@pytest.mark.parametrize("top_k", [64, 4096])
def test_decode_topk_widths_full(top_k):
    """8 sequences of 131,072 tokens with the narrowest and widest top-k
    the planner treats differently: 64 (one attention split, no merge) and
    4,096 (the largest the library takes: twice the candidates in the
    in-attention selection and 512-row splits).  Every query against the
    oracle."""
    T = 131072
    g = dict(I.GEOM_TOKEN, top_k=top_k)
    w = I.make_workload(f"k{top_k}_b8", 80 + top_k % 11, g, 8, T, np.arange(8), T - 1000 * np.arange(8))
    log(f"top-k {top_k}, 8 x 131072: workload ready")
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel_g, cnt_g = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    out_g, lse_g = dw.out.cpu().numpy(), dw.lse.cpu().numpy()
    del dw
    torch.cuda.empty_cache()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(sel_g, cnt_g, sel, cnt, f"top-k {top_k}")
    check_attention(out_g, lse_g, out, lse, f"top-k {top_k}")


def test_decode_longest_context():
    """One query over 4,194,299 of 4,194,304 cached tokens (2^22 rows of
    keys, 4.8 GB of latent cache): the top-k chunks grow to keep at most
    1,024 per query, and row indices pass 2^21.  Selection bit-exact and
    output within tolerance of the oracle."""
    T = 1 << 22
    w = I.make_workload("long4m", 90, I.GEOM_TOKEN, 1, T, [0], [T - 5])
    log("one query at 2^22 tokens: workload ready")
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel_g, cnt_g = dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy()
    out_g, lse_g = dw.out.cpu().numpy(), dw.lse.cpu().numpy()
    del dw
    torch.cuda.empty_cache()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(sel_g, cnt_g, sel, cnt, "2^22 tokens")
    check_attention(out_g, lse_g, out, lse, "2^22 tokens")
