"""One workspace serving a sequence of fused steps whose query count and
visible bound change from call to call, with no clearing in between: a
serving loop whose batch changes step to step (TensorSharp2 GLM docs,
"Serving concurrent requests": a batched decode over the concurrent
sequences, one sequence at a time when batching declines).  Every call is
compared with the oracle, and the first-digit histograms of the workspace's
histogram region must be all zero after each call."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import HIST_BLOCK, check_attention, check_selection, first_digit_dirty, hist_region, log
from oracle import oracle as O

pytestmark = pytest.mark.gpu

from deepseek_sparse_attention_amd import binding as B   # noqa: E402
from deepseek_sparse_attention_amd import inputs as I    # noqa: E402

T = 131072

# (sequences, visible tokens) of each call, in order: 8 -> 2 -> 8 -> 1 -> 4
# (short contexts: the one-kernel top-k) -> 8 (a smaller bound) -> 8
CALLS = [
    (list(range(8)), [T] * 8),
    ([5, 6], [100000, 70001]),
    (list(range(8)), [T] * 8),
    ([3], [T]),
    ([1, 2, 4, 0], [9000, 16000, 3000, 2048]),
    ([7, 6, 5, 4, 3, 2, 1, 0], [120000 - 7919 * i for i in range(8)]),
    (list(range(8)), [T] * 8),
]


def test_workspace_reused_across_batch_shapes():
    w = I.decode_128k(8)
    g = w.geom
    dev = torch.device("cuda")
    cache = torch.from_numpy(w.cache).to(dev)
    idx_k = torch.from_numpy(w.idx_k).to(dev)
    ws = B.new_workspace(g, 8, T, device=dev)
    assert hist_region(ws.numel()) >= 8 * HIST_BLOCK
    sel_ld = g["top_k"] + g["kpool"] - 1
    for k, (seqs, nvis) in enumerate(CALLS):
        n_q = len(seqs)
        log(f"call {k}: n_q={n_q}, max_nvis={max(nvis)}")
        qs = np.asarray(seqs, np.int32)
        nv = np.asarray(nvis, np.int32)
        q_seq = torch.from_numpy(qs).to(dev)
        q_nvis = torch.from_numpy(nv).to(dev)
        # query j of this call is the workload's query of its sequence
        q = torch.from_numpy(np.ascontiguousarray(w.q[qs])).to(dev)
        iq = torch.from_numpy(np.ascontiguousarray(w.idx_q[qs])).to(dev)
        iw = torch.from_numpy(np.ascontiguousarray(w.idx_w[qs])).to(dev)
        sel = torch.full((n_q, sel_ld), -7, dtype=torch.int32, device=dev)
        cnt = torch.empty(n_q, dtype=torch.int32, device=dev)
        out = torch.empty((n_q, g["n_heads"], g["d_latent"]), dtype=torch.float32, device=dev)
        lse = torch.empty((n_q, g["n_heads"]), dtype=torch.float32, device=dev)
        b = B.batch(q_seq, q_nvis, int(nv.max()), 8)
        B.decode_step(g, b, iq, iw, idx_k, w.key_rows, q, cache, T, sel, sel_ld, cnt, out, lse, ws)
        torch.cuda.synchronize()
        assert first_digit_dirty(ws) == 0, f"call {k}: histogram region left dirty"
        rsel, rcnt, rout, rlse = O.decode_step(g, qs, nv, w.idx_q[qs], w.idx_w[qs], w.idx_k, w.q[qs], w.cache)
        check_selection(sel.cpu().numpy(), cnt.cpu().numpy(), rsel, rcnt, f"call {k}")
        check_attention(out.cpu().numpy(), lse.cpu().numpy(), rout, rlse, f"call {k}")


def test_workspace_too_small_for_the_call_is_refused():
    """A call whose shape does not fit the workspace it is given is refused
    before anything runs (here: a workspace sized for 2 queries, a call of 8)."""
    w = I.make_workload("ws_small", 77, I.GEOM_TOKEN, 8, 5000, np.arange(8), [5000] * 8)
    g = w.geom
    dev = torch.device("cuda")
    ws = B.new_workspace(g, 2, 5000, device=dev)
    t = {k: torch.from_numpy(getattr(w, k)).to(dev) for k in ("cache", "idx_k", "q", "idx_q", "idx_w")}
    out = torch.full((8, 64, 512), 3.0, device=dev)
    b = B.batch(None, torch.from_numpy(w.q_nvis).to(dev), 5000, 8)
    with pytest.raises(B.DSAError) as e:
        B.decode_step(g, b, t["idx_q"], t["idx_w"], t["idx_k"], w.key_rows, t["q"], t["cache"], w.T, None,
                      2048, None, out, None, ws)
    assert e.value.status == B.DSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


@pytest.mark.parametrize("path", ["fused", "select"])
@pytest.mark.parametrize("T", [40000, 9000])
def test_garbage_workspace_is_survived_and_cleared(T, path, monkeypatch):
    """A workspace whose every byte is random breaks the rule that its
    first-digit histograms are zero between calls.  Every top-k path reads
    them (the chunked top-k at T = 40,000; at T = 9,000 k_select, or the
    fused step's one-pass top-k, which takes the scorer's histogram when
    the attention is split), so the first call's selection is meaningless,
    but every row it reads still lies in the caches, so it completes, and it
    clears its queries' histograms, so the next call of the same shape on
    that workspace is exact."""
    monkeypatch.setenv("DSA_ATTN_SEL", "1" if path == "fused" else "0")
    w = I.make_workload(f"ws_garbage_{T}", 91, I.GEOM_TOKEN, 2, T, np.arange(2), [T, T - 1234])
    g = w.geom
    dev = torch.device("cuda")
    ws = B.new_workspace(g, 2, T, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(T + (path == "fused"))
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=dev, generator=gen))
    t = {k: torch.from_numpy(getattr(w, k)).to(dev) for k in ("cache", "idx_k", "q", "idx_q", "idx_w")}
    sel_ld = g["top_k"] + g["kpool"] - 1
    b = B.batch(None, torch.from_numpy(w.q_nvis).to(dev), int(w.q_nvis.max()), 2)
    rsel, rcnt, rout, rlse = O.decode_step(g, w.q_seq, w.q_nvis, w.idx_q, w.idx_w, w.idx_k, w.q, w.cache)
    for k in range(2):
        log(f"garbage workspace T={T} {path}: call {k}")
        sel = torch.full((2, sel_ld), -7, dtype=torch.int32, device=dev)
        cnt = torch.empty(2, dtype=torch.int32, device=dev)
        out = torch.empty((2, g["n_heads"], g["d_latent"]), dtype=torch.float32, device=dev)
        lse = torch.empty((2, g["n_heads"]), dtype=torch.float32, device=dev)
        B.decode_step(g, b, t["idx_q"], t["idx_w"], t["idx_k"], w.key_rows, t["q"], t["cache"], w.T, sel, sel_ld,
                      cnt, out, lse, ws)
        torch.cuda.synchronize()
        if k == 1:
            check_selection(sel.cpu().numpy(), cnt.cpu().numpy(), rsel, rcnt, f"T={T} {path}")
            check_attention(out.cpu().numpy(), lse.cpu().numpy(), rout, rlse, f"T={T} {path}")
