"""The allocation-free fused step (dsa_decode_step_noalloc, on the library's
own device scratch) against the fused step on a caller workspace: two calls
in a row, the second smaller than the first, each bit-identical to the
workspace call and within the parity bar of the oracle; then a call too
large for the scratch, refused before anything runs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import check_attention, check_selection, log, oracle_decode

pytestmark = pytest.mark.gpu

from deepseek_sparse_attention_amd import binding as B            # noqa: E402
from deepseek_sparse_attention_amd import inputs as I             # noqa: E402
from deepseek_sparse_attention_amd.workload import DeviceWorkload  # noqa: E402


def _noalloc(dw):
    sel = torch.full_like(dw.sel, -9)
    cnt = torch.full_like(dw.sel_count, -9)
    out = torch.full_like(dw.out, float("nan"))
    lse = torch.full_like(dw.lse, float("nan"))
    B.decode_step_noalloc(dw.geom, dw.batch, dw.idx_q, dw.idx_w, dw.idx_k, dw.w.key_rows, dw.q, dw.cache, dw.w.T,
                          sel, dw.sel_ld, cnt, out, lse)
    return sel, cnt, out, lse


def test_noalloc_matches_the_workspace_call():
    big = I.decode_128k(8)
    small = I.make_workload("noalloc_small", 91, I.GEOM_TOKEN, 2, 5003, [0, 1, 1], [5003, 4097, 1500])
    for name, w in (("8 x 131072", big), ("3 queries, 5003", small)):
        log(f"noalloc {name}")
        dw = DeviceWorkload(w)
        sel, cnt, out, lse = _noalloc(dw)
        dw.decode_step()
        torch.cuda.synchronize()
        assert torch.equal(sel, dw.sel) and torch.equal(cnt, dw.sel_count), f"{name}: selection differs"
        assert torch.equal(out, dw.out) and torch.equal(lse, dw.lse), f"{name}: output differs"
        rsel, rcnt, rout, rlse = oracle_decode(w)
        check_selection(sel.cpu().numpy(), cnt.cpu().numpy(), rsel, rcnt, f"noalloc {name}")
        check_attention(out.cpu().numpy(), lse.cpu().numpy(), rout, rlse, f"noalloc {name}")
        del dw
        torch.cuda.empty_cache()


def test_noalloc_refuses_a_call_beyond_its_scratch():
    g = I.GEOM_TOKEN
    n_q, T = 8, 1 << 20
    assert B.workspace_bytes(g, n_q, T) > 32 << 20
    dev = "cuda"
    # tiny stand-ins: the call is refused on its sizes before any pointer is read
    t16 = torch.zeros(16, dtype=torch.int16, device=dev)
    tf = torch.zeros(16, dtype=torch.float32, device=dev)
    out = torch.full((8, 16), 5.0, device=dev)
    b = B.batch(None, torch.full((n_q,), T, dtype=torch.int32, device=dev), T, n_q)
    with pytest.raises(B.DSAError) as e:
        B.decode_step_noalloc(g, b, t16, tf, t16, T, t16, t16, T, None, 2048, None, out, None)
    assert e.value.status == B.DSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
