"""Selection around the budget, on the GPU: every visible count from three
rows below the keep budget to four pools above it (kpool 1: tokens, kpool
4: pools plus every tail length), for small and full-size top-k, with
all-equal and two-valued scores, where the dense/sparse switch and the tie
rule decide everything.  Through the standalone top-k on given scores and
through the fused step on keys built to give such scores, on both select
paths, bit-exact against the oracle.  (Strata PR, verification notes on the
selection rewrite: every pool count and selection width that straddles the
budget; "GLM-5.3-Flash on WASTE", "What is checked": the sparse branch must
actually be reached.)"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

from gpu_common import check_attention, check_selection, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu

from deepseek_sparse_attention_amd import binding as B            # noqa: E402
from deepseek_sparse_attention_amd import inputs as I             # noqa: E402
from deepseek_sparse_attention_amd.workload import DeviceWorkload  # noqa: E402

PAIRS = [(1, 7), (1, 2048), (4, 16), (4, 2048)]
BF16_ONE = 0x3F80


def geom(kpool, top_k):
    return dict(I.GEOM_TOKEN if kpool == 1 else I.GEOM_KPOOL, top_k=top_k)


def straddle(kpool, top_k):
    """n_vis from (keep - 3) kpool to (keep + 4) kpool + 3, keep = top_k / kpool."""
    keep = top_k // kpool
    return np.arange((keep - 3) * kpool, (keep + 4) * kpool + 4, dtype=np.int32)


def two_valued(kind, shape, seed):
    rng = np.random.default_rng(seed)
    if kind == "equal":
        return np.zeros(shape, bool)
    return rng.random(shape) < 0.5


@pytest.mark.parametrize("select", ["scan", "chunked"])
@pytest.mark.parametrize("kind", ["equal", "two"])
@pytest.mark.parametrize("kpool,top_k", PAIRS)
def test_topk_straddles_the_budget(kpool, top_k, kind, select, monkeypatch):
    monkeypatch.setenv("DSA_SELECT_SCAN", "1" if select == "scan" else "0")
    g = geom(kpool, top_k)
    nvis = straddle(kpool, top_k)
    rows = nvis // kpool
    ld = int(rows.max())
    log(f"straddle topk kpool={kpool} k={top_k} {kind} {select}: n_vis {nvis[0]}..{nvis[-1]}")
    hi = two_valued(kind, (len(nvis), ld), zlib.crc32(f"{kpool}/{top_k}/{kind}".encode()))
    s = np.where(hi, np.float32(2.0), np.float32(1.0)).astype(np.float32)
    for j, r in enumerate(rows):
        s[j, r:] = np.nan
    sel_ref, cnt_ref = O.topk(nvis, kpool, top_k, s)
    dev = "cuda"
    b = B.batch(None, torch.from_numpy(nvis).to(dev), int(nvis.max()), len(nvis))
    ws = B.new_workspace(g, len(nvis), int(nvis.max()))
    sel_ld = top_k + kpool - 1
    sel = torch.full((len(nvis), sel_ld), -9, dtype=torch.int32, device=dev)
    cnt = torch.full((len(nvis),), -9, dtype=torch.int32, device=dev)
    B.topk(g, b, torch.from_numpy(s).to(dev), ld, sel, sel_ld, cnt, ws)
    torch.cuda.synchronize()
    check_selection(sel.cpu().numpy(), cnt.cpu().numpy(), sel_ref, cnt_ref, f"{kpool}/{top_k}/{kind}")


@pytest.mark.parametrize("select", ["scan", "chunked"])
@pytest.mark.parametrize("kind", ["equal", "two"])
@pytest.mark.parametrize("kpool,top_k", PAIRS)
def test_fused_step_straddles_the_budget(kpool, top_k, kind, select, monkeypatch):
    """The same counts through the fused step: one sequence; key rows are
    zero (score 0) or the unit vector e_0 against indexer queries whose
    first dimension is 1 for every head (score = the sum of the weights)."""
    monkeypatch.setenv("DSA_SELECT_SCAN", "1" if select == "scan" else "0")
    g = geom(kpool, top_k)
    nvis = straddle(kpool, top_k)
    T = int(nvis.max())
    log(f"straddle step kpool={kpool} k={top_k} {kind} {select}: n_vis {nvis[0]}..{nvis[-1]}")
    w = I.make_workload(f"straddle_{kpool}_{top_k}", 300 + kpool * 10 + top_k % 7, g, 1, T,
                        np.zeros(len(nvis), np.int32), nvis)
    hi = two_valued(kind, w.idx_k.shape[1], zlib.crc32(f"step/{kpool}/{top_k}/{kind}".encode()))
    w.idx_k[:] = 0
    w.idx_k[0, hi, 0] = BF16_ONE
    w.idx_q[:] = 0
    w.idx_q[:, :, 0] = BF16_ONE
    dw = DeviceWorkload(w)
    dw.sel.fill_(-9)
    dw.decode_step()
    torch.cuda.synchronize()
    sel, cnt, out, lse = O.decode_step(w.geom, w.q_seq, w.q_nvis, w.idx_q, w.idx_w, w.idx_k, w.q, w.cache)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, f"step {kpool}/{top_k}/{kind}")
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, f"step {kpool}/{top_k}/{kind}")
