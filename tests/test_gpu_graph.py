"""The fused step captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed several times, with eager work and synchronisation between the
replays: every replay must reproduce the eager call bit for bit.  The
library allocates nothing and records no memset, so its launches are
capturable as they stand."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import log, gpu_arch

pytestmark = pytest.mark.gpu

from oracle import oracle as O                                     # noqa: E402
from deepseek_sparse_attention_amd import binding as B            # noqa: E402
from deepseek_sparse_attention_amd import inputs as I             # noqa: E402
from deepseek_sparse_attention_amd.workload import DeviceWorkload  # noqa: E402


def setup_module():
    assert gpu_arch().startswith("gfx950")
    B.device_check()


# name, geometry, n_seq, T, q_seq, q_nvis: a batch that takes the chunked
# top-k (rows > 16,384), the wave-private attention with splits and the
# merge, plus a dense query and an invalid one
CASES = [
    ("tok_chunked", dict(I.GEOM_TOKEN), 4, 40000, [0, 1, 2, 3, 0], [40000, 30001, 20480, 1500, 0]),
    ("pool", dict(I.GEOM_TOKEN, kpool=4, d_rope=0), 2, 90001, [0, 1, 1], [90001, 70003, 2051]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_captured_step_replays_match_eager(case):
    name, g, n_seq, T, q_seq, q_nvis = case
    log(f"graph {name}")
    w = I.make_workload(name, 300, g, n_seq, T, q_seq, q_nvis)
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dw.sel, dw.sel_count, dw.out, dw.lse)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dw.decode_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dw.decode_step()
    torch.cuda.synchronize()

    for k in range(4):
        # eager work between the replays: poison every output
        dw.sel.fill_(-7)
        dw.sel_count.fill_(-7)
        dw.out.fill_(float("nan"))
        dw.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((dw.sel, dw.sel_count, dw.out, dw.lse), ref, ("sel", "count", "out", "lse")):
            assert torch.equal(got, want) or (what in ("out", "lse") and torch.equal(got.nan_to_num(7.0),
                                                                                  want.nan_to_num(7.0))), \
                f"{name}: replay {k}: {what} differs from the eager call"
    del graph


def test_stream_read_probe():
    """The bandwidth probe reads a buffer without writing its sink (the
    words of a constant buffer xor to zero), and refuses a size that is not
    a multiple of 16 bytes or a misaligned buffer."""
    buf = torch.full((1 << 20,), 3, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    with pytest.raises(B.DSAError):
        B.stream_read(buf[:100], sink)
    with pytest.raises(B.DSAError):
        B.stream_read(buf[1:1 + 4096], sink)


# name, geometry, n_seq, T, q_seq, q_nvis, whether the filter kernel runs
# (rows > 16,384), whether the merge runs (more than one split)
# name, geometry, n_seq, T, q_seq, q_nvis, filter runs, k_reduce runs
TIMED = [
    ("tok_chunked", dict(I.GEOM_TOKEN), 4, 40000, [0, 1, 2, 3, 0], [40000, 30001, 20480, 1500, 0], True, True),
    ("one_query_scan", dict(I.GEOM_TOKEN), 1, 9000, [0], [9000], False, True),
]


@pytest.mark.parametrize("case", TIMED, ids=[c[0] for c in TIMED])
def test_timing_events_time_the_kernels_that_ran(case):
    """With timing events set, the step gives the same outputs, reports the
    kernels it ran (the filter only for the chunked top-k, no separate select
    kernel for a decode batch), and each of them
    has a positive start-to-stop interval inside the call's own bracket."""
    name, g, n_seq, T, q_seq, q_nvis, filt, merge = case
    log(f"timing events {name}")
    w = I.make_workload(name, 301, g, n_seq, T, q_seq, q_nvis)
    dw = DeviceWorkload(w)
    dw.decode_step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dw.sel, dw.sel_count, dw.out, dw.lse)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(12)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    evs[10].record()
    B.set_timing_events(evs[:10])
    try:
        dw.decode_step()
    finally:
        B.set_timing_events(None)
    evs[11].record()
    torch.cuda.synchronize()
    ran = B.timing_ran()
    # decode batches of up to 64 queries select inside the attention kernel
    assert ran & 0b01001 == 0b01001, f"score and attend always run: {ran:#b}"
    assert not ran & 0b00100, f"no separate select kernel for a decode batch: {ran:#b}"
    assert bool(ran & 0b00010) == filt and bool(ran & 0b10000) == merge, f"{ran:#b}"
    whole = evs[10].elapsed_time(evs[11])
    for j in range(5):
        if (ran >> j) & 1:
            t0, t1 = evs[10].elapsed_time(evs[2 * j]), evs[10].elapsed_time(evs[2 * j + 1])
            assert 0.0 <= t0 < t1 <= whole, f"kernel {j}: [{t0}, {t1}] outside [0, {whole}] ms"
    for got, want in zip((dw.sel, dw.sel_count, dw.out.nan_to_num(7.0), dw.lse.nan_to_num(7.0)),
                         (ref[0], ref[1], ref[2].nan_to_num(7.0), ref[3].nan_to_num(7.0))):
        assert torch.equal(got, want)


# identity sequence maps with dense, invalid and short-tile queries: the
# scorer's early first fetch (NULL map) against the explicit map
NULL_MAP = [
    ("tok", dict(I.GEOM_TOKEN), 4, 40000, [0, 1, 2, 3], [40000, 1500, 0, 17001]),
    ("pool", dict(I.GEOM_TOKEN, kpool=4, d_rope=0), 3, 90001, [0, 1, 2], [90001, 2051, 8195]),
    ("pool_no_rows", dict(I.GEOM_TOKEN, kpool=4, d_rope=0), 2, 4, [0, 1], [3, 1]),
    ("tok_one_row", dict(I.GEOM_TOKEN), 2, 1, [0, 1], [1, 1]),
    ("tok_one_tile", dict(I.GEOM_TOKEN), 3, 3000, [0, 1, 2], [3000, 2049, 1023]),
]


@pytest.mark.parametrize("case", NULL_MAP, ids=[c[0] for c in NULL_MAP])
def test_null_sequence_map_matches_explicit_map(case):
    """A batch whose query i reads sequence i gives bit-identical results
    with q_seq NULL and with the explicit map."""
    name, g, n_seq, T, q_seq, q_nvis = case
    log(f"NULL sequence map {name}")
    w = I.make_workload(name, 303, g, n_seq, T, q_seq, q_nvis)
    a, b = DeviceWorkload(w, seq_map="auto"), DeviceWorkload(w, seq_map="always")
    assert a.batch.q_seq is None and b.batch.q_seq is not None
    for _ in range(2):
        a.decode_step()
        b.decode_step()
    torch.cuda.synchronize()
    assert torch.equal(a.sel, b.sel) and torch.equal(a.sel_count, b.sel_count)
    assert torch.equal(a.out.nan_to_num(7.0), b.out.nan_to_num(7.0))
    assert torch.equal(a.lse.nan_to_num(7.0), b.lse.nan_to_num(7.0))
    kp = g["kpool"]
    scores = O.index_scores(w.q_seq, w.q_nvis, kp, w.idx_q, w.idx_w, w.idx_k)
    sel, cnt = O.topk(w.q_nvis, kp, g["top_k"], scores)
    assert np.array_equal(a.sel_count.cpu().numpy(), cnt) and np.array_equal(a.sel.cpu().numpy(), sel)
