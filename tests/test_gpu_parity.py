"""Parity of the HIP path (through the C ABI) with the CPU oracle, at sizes
the oracle finishes in seconds: several score tiles, top-k chunks and
attention splits, ragged tails, dense and sparse queries in one batch,
token-level and k-pool geometries."""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

from gpu_common import (HIST_BLOCK, check_attention, check_selection, first_digit_dirty, gpu_arch,
                        hist_region, log, oracle_decode)
from oracle import oracle as O

pytestmark = pytest.mark.gpu

from deepseek_sparse_attention_amd import binding as B            # noqa: E402
from deepseek_sparse_attention_amd import inputs as I             # noqa: E402
from deepseek_sparse_attention_amd.workload import DeviceWorkload  # noqa: E402


def setup_module():
    arch = gpu_arch()
    log(f"device arch {arch}")
    assert arch.startswith("gfx950"), arch
    B.device_check()


# DSA_ATTN_HS value that forces each attention kernel
ATTN_KERNEL = {"wide": "0", "hs": "1", "wv": "2"}


def geom(kpool=1, d_rope=64, top_k=2048):
    g = dict(I.GEOM_TOKEN)
    g.update(kpool=kpool, d_rope=d_rope, top_k=top_k)
    return g


# name, geometry, n_seq, T, q_seq, q_nvis, key range
CASES = [
    ("tok_mixed", geom(), 2, 5003, [0, 1, 1, 0], [5003, 4097, 1500, 2049], (-8, 8)),
    ("tok_ties", geom(), 1, 6000, [0, 0], [6000, 3001], (-1, 1)),
    ("tok_k64", geom(top_k=64), 2, 3000, [1, 0, 1], [3000, 65, 64], (-8, 8)),
    ("tok_k1", geom(top_k=1), 1, 1200, [0, 0], [1200, 1], (-8, 8)),
    ("tok_k4096", geom(top_k=4096), 1, 9000, [0], [9000], (-8, 8)),
    ("pool_mixed", geom(kpool=4, d_rope=0), 2, 12301, [0, 1, 1], [12301, 2051, 2052], (-8, 8)),
    ("pool_k16", geom(kpool=4, d_rope=0, top_k=16), 1, 4099, [0, 0, 0], [4099, 19, 20], (-8, 8)),
    ("pool_rope", geom(kpool=4, d_rope=64), 1, 9002, [0], [9002], (-4, 4)),
    ("tok_nope", geom(kpool=1, d_rope=0), 1, 4500, [0], [4500], (-8, 8)),
]


def make_case(i, name, g, n_seq, T, q_seq, q_nvis, kr):
    return I.make_workload(name, 100 + i, g, n_seq, T, q_seq, q_nvis, key_range=kr)


@pytest.mark.parametrize("scorer", ["mfma", "valu"])
@pytest.mark.parametrize("case", list(enumerate(CASES)), ids=[c[0] for c in CASES])
def test_scores_bit_exact(case, scorer, monkeypatch):
    """Scores of the MFMA scorer and of its vector-ALU variant (kept to
    measure the two against each other), bit for bit."""
    if scorer == "valu":
        monkeypatch.setenv("DSA_SCORE_VALU", "1")
    i, (name, g, n_seq, T, q_seq, q_nvis, kr) = case
    log(f"scores {name} ({scorer})")
    w = make_case(i, name, g, n_seq, T, q_seq, q_nvis, kr)
    dw = DeviceWorkload(w)
    rows_max = dw.max_nvis // g["kpool"]
    ld = rows_max + 5
    scores = torch.full((w.n_q, ld), float("nan"), device="cuda")
    B.index_scores(g, dw.batch, dw.idx_q, dw.idx_w, dw.idx_k, w.key_rows, scores, ld)
    torch.cuda.synchronize()
    ref = O.index_scores(w.q_seq, w.q_nvis, g["kpool"], w.idx_q, w.idx_w, w.idx_k, score_ld=ld)
    got = scores.cpu().numpy()
    for j in range(w.n_q):
        rows = int(w.q_nvis[j]) // g["kpool"]
        assert np.array_equal(got[j, :rows], ref[j, :rows]), f"{name} q{j}"
        assert np.isnan(got[j, rows:]).all(), f"{name} q{j} wrote past rows"


# fused-step paths for a decode batch: the top-k inside the attention kernel
# (default), or k_select + the attention kernel
PATHS = {"fused": {}, "select": {"DSA_ATTN_SEL": "0"}}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", list(enumerate(CASES)), ids=[c[0] for c in CASES])
def test_decode_step_matches_oracle(case, path, monkeypatch):
    for k, v in PATHS[path].items():
        monkeypatch.setenv(k, v)
    i, (name, g, n_seq, T, q_seq, q_nvis, kr) = case
    log(f"decode {name} ({path})")
    w = make_case(i, name, g, n_seq, T, q_seq, q_nvis, kr)
    dw = DeviceWorkload(w)
    dw.sel.fill_(-7)
    dw.decode_step()
    torch.cuda.synchronize()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, name)
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, name)
    # the first-digit histograms of the histogram region (the workspace's
    # first sixteenth, in whole per-query blocks) are all zero again after
    # the call (workspace contract)
    assert hist_region(dw.ws.numel()) >= w.n_q * HIST_BLOCK
    assert first_digit_dirty(dw.ws) == 0, f"{name}: histogram left dirty"
    # a second call on the same workspace gives the same result bit for bit
    out1, sel1 = dw.out.clone(), dw.sel.clone()
    dw.decode_step()
    torch.cuda.synchronize()
    assert torch.equal(dw.sel, sel1) and torch.equal(dw.out, out1), f"{name}: second call differs"


def _scores_case(rng, kind, n):
    if kind == "real":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "ties":
        return rng.integers(0, 5, n).astype(np.float32)
    if kind == "zeros":
        return np.zeros(n, np.float32)
    if kind == "signed_zero":
        s = np.where(rng.random(n) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        s[rng.choice(n, min(100, n // 2), replace=False)] = 1.0
        return s
    if kind == "negative":
        return -rng.integers(0, 1000, n).astype(np.float32)
    raise KeyError(kind)


@pytest.mark.parametrize("kind", ["real", "ties", "zeros", "signed_zero", "negative"])
@pytest.mark.parametrize("kpool,top_k", [(1, 2048), (1, 7), (4, 2048), (4, 16)])
@pytest.mark.parametrize("select", ["scan", "chunked"])
def test_topk_bit_exact(kind, kpool, top_k, select, monkeypatch):
    """Standalone top-k on given scores, including a tie storm larger than the
    candidate buffer (all-zero scores over 20000 rows) and -0.0 / +0.0, by
    both select paths (one kernel scanning the scores, or k_filter's chunk
    slots gathered by k_select)."""
    monkeypatch.setenv("DSA_SELECT_SCAN", "1" if select == "scan" else "0")
    log(f"topk {kind} kpool={kpool} k={top_k} select={select}")
    rng = np.random.default_rng(zlib.crc32(f"{kind}/{kpool}/{top_k}".encode()))
    g = geom(kpool=kpool, d_rope=0 if kpool == 4 else 64, top_k=top_k)
    nvis = np.array([80003, 20000, top_k + kpool - 1, top_k + kpool, 5], np.int32)
    rows = nvis // kpool
    ld = int(rows.max())
    s = np.stack([np.pad(_scores_case(rng, kind, int(r)), (0, ld - int(r)), constant_values=np.nan)
                  for r in rows]).astype(np.float32)
    sel_ref, cnt_ref = O.topk(nvis, kpool, top_k, s)
    dev = "cuda"
    q_nvis = torch.from_numpy(nvis).to(dev)
    b = B.batch(None, q_nvis, int(nvis.max()), len(nvis))
    ws = B.new_workspace(g, len(nvis), int(nvis.max()))
    sel_ld = top_k + kpool - 1
    sel = torch.full((len(nvis), sel_ld), -9, dtype=torch.int32, device=dev)
    cnt = torch.full((len(nvis),), -9, dtype=torch.int32, device=dev)
    st = torch.from_numpy(s).to(dev)
    B.topk(g, b, st, ld, sel, sel_ld, cnt, ws)
    torch.cuda.synchronize()
    check_selection(sel.cpu().numpy(), cnt.cpu().numpy(), sel_ref, cnt_ref, f"{kind}/{kpool}/{top_k}")
    # twice in a row on the same workspace
    B.topk(g, b, st, ld, sel, sel_ld, cnt, ws)
    torch.cuda.synchronize()
    check_selection(sel.cpu().numpy(), cnt.cpu().numpy(), sel_ref, cnt_ref, f"{kind}/{kpool}/{top_k} again")


@pytest.mark.parametrize("d_rope", [64, 0])
@pytest.mark.parametrize("count", [1, 31, 32, 33, 100, 2048, 2051])
@pytest.mark.parametrize("kernel", ["hs", "wv", "wide"])
def test_attend_matches_oracle(d_rope, count, kernel, monkeypatch):
    """The three attention kernels (head-split, wave-private rows, and all
    heads per work-group), forced by the planner's override, against the
    oracle."""
    monkeypatch.setenv("DSA_ATTN_HS", ATTN_KERNEL[kernel])
    log(f"attend d_rope={d_rope} count={count} kernel={kernel}")
    rng = np.random.default_rng(count * 7 + d_rope)
    g = geom(kpool=4 if d_rope == 0 else 1, d_rope=d_rope)
    D = 512 + d_rope
    T = 6000
    cache = I.f32_to_bf16_bits(rng.standard_normal((2, T, D)).astype(np.float32))
    n_q = 3
    q = I.f32_to_bf16_bits(rng.standard_normal((n_q, 64, D)).astype(np.float32))
    q_seq = np.array([0, 1, 1], np.int32)
    sel_ld = g["top_k"] + g["kpool"] - 1
    sel = np.full((n_q, sel_ld), -1, np.int32)
    cnt = np.zeros(n_q, np.int32)
    for j in range(n_q):
        c = min(count, sel_ld)
        sel[j, :c] = np.sort(rng.choice(T, c, replace=False))
        cnt[j] = c
    out_ref, lse_ref = O.mla_attend(q_seq, 512, d_rope, 1 / 16, q, cache, sel, cnt)
    dev = "cuda"
    b = B.batch(torch.from_numpy(q_seq).to(dev), torch.full((n_q,), T, dtype=torch.int32, device=dev), T, 2)
    ws = B.new_workspace(g, n_q, T)
    out = torch.full((n_q, 64, 512), float("nan"), device=dev)
    lse = torch.full((n_q, 64), float("nan"), device=dev)
    B.mla_attend(g, b, torch.from_numpy(q).to(dev), torch.from_numpy(cache).to(dev), T,
                 torch.from_numpy(sel).to(dev), sel_ld, torch.from_numpy(cnt).to(dev), out, lse, ws)
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), out_ref, lse_ref, f"attend D={D} n={count}")


def _attend_case(d_rope, n_q, sel, cnt, T, seed):
    rng = np.random.default_rng(seed)
    g = geom(kpool=4 if d_rope == 0 else 1, d_rope=d_rope)
    D = 512 + d_rope
    cache = I.f32_to_bf16_bits(rng.standard_normal((2, T, D)).astype(np.float32))
    q = I.f32_to_bf16_bits(rng.standard_normal((n_q, 64, D)).astype(np.float32))
    q_seq = (np.arange(n_q) % 2).astype(np.int32)
    sel_ld = sel.shape[1]
    dev = "cuda"
    b = B.batch(torch.from_numpy(q_seq).to(dev), torch.full((n_q,), T, dtype=torch.int32, device=dev), T, 2)
    ws = B.new_workspace(g, n_q, T)
    out = torch.full((n_q, 64, 512), 7.0, device=dev)
    lse = torch.full((n_q, 64), 7.0, device=dev)
    B.mla_attend(g, b, torch.from_numpy(q).to(dev), torch.from_numpy(cache).to(dev), T,
                 torch.from_numpy(sel).to(dev), sel_ld, torch.from_numpy(cnt).to(dev), out, lse, ws)
    torch.cuda.synchronize()
    return g, q_seq, q, cache, out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("d_rope", [64, 0])
@pytest.mark.parametrize("kernel", ["hs", "wv", "wide"])
def test_attend_skips_invalid_rows_and_counts(d_rope, kernel, monkeypatch):
    """Entries outside [0, T) inside the count are skipped; a count outside
    [0, top_k + kpool - 1], or one that leaves no row, gives NaN."""
    monkeypatch.setenv("DSA_ATTN_HS", ATTN_KERNEL[kernel])
    log(f"attend edge rows d_rope={d_rope} kernel={kernel}")
    rng = np.random.default_rng(91 + d_rope)
    T, n_q = 3000, 8
    kp = 4 if d_rope == 0 else 1
    sel_ld = 2048 + kp - 1
    sel = np.full((n_q, sel_ld), -1, np.int32)
    cnt = np.zeros(n_q, np.int32)
    for j in range(n_q):
        c = [700, 1500, 40, 2048 + kp - 1, 64, 5, 10, 300][j]
        sel[j, :c] = np.sort(rng.choice(T, c, replace=False))
        cnt[j] = c
    sel[0, [3, 100, 650]] = -1            # skipped
    sel[1, [0, 777]] = [T + 5, 2 ** 30]   # beyond the cache rows: skipped
    cnt[4] = sel_ld + 1                   # too many: NaN
    cnt[5] = -3                           # negative: NaN
    sel[6, :10] = -1                      # nothing left: NaN
    cnt[7] = 0                            # empty: NaN
    g, q_seq, q, cache, out, lse = _attend_case(d_rope, n_q, sel, cnt, T, 5 + d_rope)
    for j in range(4):
        rows = sel[j, :cnt[j]]
        rows = rows[(rows >= 0) & (rows < T)]
        s1 = np.full((1, sel_ld), -1, np.int32)
        s1[0, :len(rows)] = rows
        o_ref, l_ref = O.mla_attend(q_seq[j:j + 1], 512, d_rope, 1 / 16, q[j:j + 1], cache, s1,
                                    np.array([len(rows)], np.int32))
        check_attention(out[j:j + 1], lse[j:j + 1], o_ref, l_ref, f"edge q{j}")
    for j in range(4, 8):
        assert np.isnan(out[j]).all() and np.isnan(lse[j]).all(), f"query {j} should be NaN"


@pytest.mark.parametrize("pairs", [None, "4"])
@pytest.mark.parametrize("d_rope", [64, 0])
@pytest.mark.parametrize("kernel", ["hs", "wv", "wide"])
def test_attend_rising_scores(kernel, d_rope, pairs, monkeypatch):
    """Scores that rise by ~11.5 log2 units from one 16-row step of a wave
    to its next: every kernel must move its softmax reference many times
    (k_attend_wv restarts its rows each time).  The scores are integers
    (queries 1 on the first 64 dimensions, cache entries integer there), so
    they are exact in any summation order; with pairs = 4 every query is one
    2048-row split."""
    monkeypatch.setenv("DSA_ATTN_HS", ATTN_KERNEL[kernel])
    if pairs:
        monkeypatch.setenv("DSA_ATTN_PAIRS", pairs)
    log(f"attend rising scores kernel={kernel} d_rope={d_rope} pairs={pairs}")
    rng = np.random.default_rng(41 + d_rope)
    g = geom(kpool=4 if d_rope == 0 else 1, d_rope=d_rope)
    D = 512 + d_rope
    T, n_q = 6000, 4
    sel_ld = g["top_k"] + g["kpool"] - 1
    cache = rng.standard_normal((2, T, D)).astype(np.float32)
    q = np.zeros((n_q, 64, D), np.float32)
    q[:, :, :64] = 1.0
    q_seq = (np.arange(n_q) % 2).astype(np.int32)
    sel = np.full((n_q, sel_ld), -1, np.int32)
    cnt = np.full(n_q, 2048, np.int32)
    for j in range(n_q):
        rows = np.sort(rng.choice(T, 2048, replace=False))
        sel[j, :2048] = rows
        # the p-th selected row scores 64 * 2 * (p // 64)
        cache[q_seq[j], rows, :64] = (2 * (np.arange(2048) // 64))[:, None]
    cache = I.f32_to_bf16_bits(cache)
    q = I.f32_to_bf16_bits(q)
    out_ref, lse_ref = O.mla_attend(q_seq, 512, d_rope, 1 / 16, q, cache, sel, cnt)
    dev = "cuda"
    b = B.batch(torch.from_numpy(q_seq).to(dev), torch.full((n_q,), T, dtype=torch.int32, device=dev), T, 2)
    ws = B.new_workspace(g, n_q, T)
    out = torch.full((n_q, 64, 512), float("nan"), device=dev)
    lse = torch.full((n_q, 64), float("nan"), device=dev)
    B.mla_attend(g, b, torch.from_numpy(q).to(dev), torch.from_numpy(cache).to(dev), T,
                 torch.from_numpy(sel).to(dev), sel_ld, torch.from_numpy(cnt).to(dev), out, lse, ws)
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), out_ref, lse_ref, f"rising D={D}")


@pytest.mark.parametrize("kernel", ["hs", "wv", "wide"])
def test_attend_single_split_path(kernel, monkeypatch):
    """Many queries: every query is one work-group (or four head groups)
    that writes its output directly (no split merge)."""
    monkeypatch.setenv("DSA_ATTN_HS", ATTN_KERNEL[kernel])
    log(f"attend single split kernel={kernel}")
    rng = np.random.default_rng(17)
    T, n_q = 2500, 300
    sel_ld = 2048
    sel = np.full((n_q, sel_ld), -1, np.int32)
    cnt = rng.integers(1, 97, n_q).astype(np.int32)
    cnt[:3] = [1, 32, 96]
    for j in range(n_q):
        sel[j, :cnt[j]] = np.sort(rng.choice(T, cnt[j], replace=False))
    g, q_seq, q, cache, out, lse = _attend_case(64, n_q, sel, cnt, T, 23)
    o_ref, l_ref = O.mla_attend(q_seq, 512, 64, 1 / 16, q, cache, sel, cnt)
    check_attention(out, lse, o_ref, l_ref, "single split")


def test_prefill_chunk_small():
    """Chunked prefill at positions 0..511 of a 4096-token context: early
    queries keep all their candidates, later ones select."""
    log("prefill c3s")
    w = I.c3_small()
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, "c3s")
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, "c3s")


def test_prefill_chunk_sparse_small():
    """Prefill chunk past the budget: 300 positions at the end of 6000."""
    log("prefill tail chunk")
    T = 6000
    pos = np.arange(T - 300, T)
    w = I.make_workload("pf", 14, I.GEOM_TOKEN, 1, T, np.zeros(300), pos + 1)
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, "prefill tail")
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, "prefill tail")


def test_prefill_runs_with_mixed_sequences():
    """Prefill batches (runs of 8 queries sharing a sequence) where one run
    mixes sequences: the dense contraction covers the run leader's
    sequence, the fix-up pass the others; both standalone and fused."""
    log("prefill mixed runs")
    T = 5000
    q_seq = [0] * 8 + [1, 1, 0, 1, 1, 1, 0, 1] + [1] * 4
    pos = [T - 20 + i for i in range(8)] + [4000 + 37 * i for i in range(8)] + [2100, 2200, 2300, 4999]
    w = I.make_workload("pfm", 15, I.GEOM_TOKEN, 2, T, q_seq, [p + 1 for p in pos])
    dw = DeviceWorkload(w)
    dw.batch = B.batch(dw.q_seq, dw.q_nvis, dw.max_nvis, w.n_seq, 8)
    ld = dw.max_nvis + 3
    scores = torch.full((w.n_q, ld), float("nan"), device="cuda")
    B.index_scores(w.geom, dw.batch, dw.idx_q, dw.idx_w, dw.idx_k, w.key_rows, scores, ld)
    dw.decode_step()
    torch.cuda.synchronize()
    ref = O.index_scores(w.q_seq, w.q_nvis, 1, w.idx_q, w.idx_w, w.idx_k, score_ld=ld)
    got = scores.cpu().numpy()
    for j in range(w.n_q):
        rows = int(w.q_nvis[j])
        assert np.array_equal(got[j, :rows], ref[j, :rows]), f"query {j}"
        assert np.isnan(got[j, rows:]).all(), f"query {j} wrote past rows"
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, "prefill mixed")
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, "prefill mixed")


@pytest.mark.parametrize("window", [2, 3, 5, 8, 9])
def test_verify_window_matches_oracle(window):
    """Speculative verify windows: B sequences x `window` rows at the last
    positions; each run of rows shares its key tiles in the prefill scorer.
    Scores bit-exact, selections bit-exact, attention within tolerance."""
    log(f"verify window {window}")
    w = I.decode_window(3, window, T=6000)
    dw = DeviceWorkload(w)
    assert dw.batch.q_per_seq_hint == window
    ld = dw.max_nvis + 1
    scores = torch.full((w.n_q, ld), float("nan"), device="cuda")
    B.index_scores(w.geom, dw.batch, dw.idx_q, dw.idx_w, dw.idx_k, w.key_rows, scores, ld)
    dw.decode_step()
    torch.cuda.synchronize()
    ref = O.index_scores(w.q_seq, w.q_nvis, 1, w.idx_q, w.idx_w, w.idx_k, score_ld=ld)
    got = scores.cpu().numpy()
    for j in range(w.n_q):
        rows = int(w.q_nvis[j])
        assert np.array_equal(got[j, :rows], ref[j, :rows]), f"query {j}"
        assert np.isnan(got[j, rows:]).all(), f"query {j} wrote past rows"
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, f"window {window}")
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, f"window {window}")


def test_run_hint_that_does_not_match_the_runs():
    """A run-length hint that disagrees with the real runs (and a query count
    that is not a multiple of it) still gives exact results: queries outside
    their block leader's sequence go through the fix-up pass."""
    log("mismatched run hint")
    T = 4000
    q_seq = [0, 0, 0, 1, 1, 1, 2, 2, 0, 1, 2]
    nvis = [3990, 3991, 3992, 2500, 2501, 2502, 3999, 4000, 1000, 3500, 2049]
    w = I.make_workload("hint", 16, I.GEOM_TOKEN, 3, T, q_seq, nvis)
    dw = DeviceWorkload(w)
    for hint in (4, 16):
        dw.batch = B.batch(dw.q_seq, dw.q_nvis, dw.max_nvis, w.n_seq, hint)
        dw.decode_step()
        torch.cuda.synchronize()
        sel, cnt, out, lse = oracle_decode(w)
        check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, f"hint {hint}")
        check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, f"hint {hint}")


@pytest.mark.parametrize("scale,kpool", [(1 / 24, 1), (1 / 512 ** 0.5, 1), (0.125, 4), (1 / 40, 4)])
def test_softmax_scales(scale, kpool):
    """Softmax scales other than the pages' 1/16 (the ABI takes any finite
    positive scale) through the fused step and the standalone attention."""
    log(f"scale {scale:.5f} kpool={kpool}")
    g = dict(geom(kpool=kpool, d_rope=0 if kpool == 4 else 64), softmax_scale=scale)
    w = I.make_workload(f"scale_{kpool}", 400 + kpool, g, 2, 9003, [0, 1, 1], [9003, 4097, 1500])
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, f"scale {scale}")
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, f"step scale {scale}")
    # the standalone attention on the oracle's selection
    out2 = torch.full_like(dw.out, float("nan"))
    lse2 = torch.full_like(dw.lse, float("nan"))
    B.mla_attend(g, dw.batch, dw.q, dw.cache, w.T, torch.from_numpy(sel).cuda(), sel.shape[1],
                 torch.from_numpy(cnt).cuda(), out2, lse2, dw.ws)
    torch.cuda.synchronize()
    out_r, lse_r = O.mla_attend(w.q_seq, 512, g["d_rope"], scale, w.q, w.cache, sel, cnt)
    check_attention(out2.cpu().numpy(), lse2.cpu().numpy(), out_r, lse_r, f"attend scale {scale}")
