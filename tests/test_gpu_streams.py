"""Concurrent fused steps on two streams, each with its own workspace (the
contract for calls on different streams): the library keeps no device
state outside the caller's workspace and outputs, so two different batches
launched back to back on two streams, their kernels free to overlap, must
give bit for bit what each gives alone, and match the oracle.  Both streams
keep the default priority."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import check_attention, check_selection, gpu_arch, log, oracle_decode

pytestmark = pytest.mark.gpu

from deepseek_sparse_attention_amd import binding as B            # noqa: E402
from deepseek_sparse_attention_amd import inputs as I             # noqa: E402
from deepseek_sparse_attention_amd.workload import DeviceWorkload  # noqa: E402


def setup_module():
    assert gpu_arch().startswith("gfx950")
    B.device_check()


def _outputs(dw):
    return dw.sel.clone(), dw.sel_count.clone(), dw.out.clone(), dw.lse.clone()


def test_two_streams_match_their_solo_runs():
    # an 8-query batch (fused top-k in the attention) and a 12-query batch
    # (k_select, then the wave-private attention), different contexts
    wa = I.make_workload("streams_a", 601, I.GEOM_TOKEN, 8, 50000, np.arange(8), 50000 - 313 * np.arange(8))
    wb = I.make_workload("streams_b", 602, I.GEOM_TOKEN, 4, 70001, np.arange(12) % 4, 70001 - 911 * np.arange(12))
    da, db = DeviceWorkload(wa), DeviceWorkload(wb)
    da.decode_step()
    db.decode_step()
    torch.cuda.synchronize()
    solo_a, solo_b = _outputs(da), _outputs(db)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for k in range(6):
        log(f"two streams, round {k}")
        for d in (da, db):
            d.sel.fill_(-7)
            d.out.fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(3):   # several steps queued on each stream
            da.decode_step(stream=sa)
            db.decode_step(stream=sb)
        torch.cuda.synchronize()
        for got, ref, name in ((_outputs(da), solo_a, "a"), (_outputs(db), solo_b, "b")):
            for x, y in zip(got, ref):
                assert torch.equal(x, y), f"round {k}: batch {name} differs from its solo run"
    for d, w, name in ((da, wa, "a"), (db, wb, "b")):
        sel, cnt, out, lse = oracle_decode(w)
        check_selection(d.sel.cpu().numpy(), d.sel_count.cpu().numpy(), sel, cnt, f"streams {name}")
        check_attention(d.out.cpu().numpy(), d.lse.cpu().numpy(), out, lse, f"streams {name}")
