"""Shared helpers of the GPU parity tests."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import oracle as O

ATTN_TOL = 2e-3       # max |o - o_ref| / max_j |o_ref[q, h, j]|
LSE_TOL = 1e-4        # absolute, natural-log units


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """Largest error of a query head's output relative to that row's largest
    magnitude (the tolerance metric of the parity bar)."""
    out = out.astype(np.float64)
    ref = ref.astype(np.float64)
    norm = np.abs(ref).max(axis=-1, keepdims=True)
    norm = np.maximum(norm, 1e-30)
    return float((np.abs(out - ref) / norm).max())


def oracle_decode(w, queries=None):
    """Oracle of the fused step for all (or a subset of) the queries."""
    idx = np.arange(w.n_q) if queries is None else np.asarray(queries)
    return O.decode_step(w.geom, w.q_seq[idx], w.q_nvis[idx], w.idx_q[idx], w.idx_w[idx], w.idx_k,
                         w.q[idx], w.cache)


def check_selection(sel_gpu, cnt_gpu, sel_ref, cnt_ref, what=""):
    sel_gpu = np.asarray(sel_gpu)
    cnt_gpu = np.asarray(cnt_gpu)
    assert np.array_equal(cnt_gpu, cnt_ref), f"{what}: counts {cnt_gpu[:8]} vs {cnt_ref[:8]}"
    for j in range(len(cnt_ref)):
        if not np.array_equal(sel_gpu[j], sel_ref[j]):
            bad = np.nonzero(sel_gpu[j] != sel_ref[j])[0]
            raise AssertionError(f"{what}: query {j} selection differs at {bad[:8]}: "
                                 f"gpu {sel_gpu[j][bad[:8]]} ref {sel_ref[j][bad[:8]]}")


def check_attention(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    err = row_rel_err(np.asarray(out_gpu), out_ref)
    lerr = float(np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref).max())
    log(f"{what}: attention row-rel err {err:.3e}, lse abs err {lerr:.3e}")
    assert np.isfinite(np.asarray(out_gpu)).all(), f"{what}: non-finite output"
    assert err <= ATTN_TOL, f"{what}: attention error {err:.3e} > {ATTN_TOL}"
    assert lerr <= LSE_TOL, f"{what}: lse error {lerr:.3e} > {LSE_TOL}"
    return err


def gpu_arch() -> str:
    return torch.cuda.get_device_properties(0).gcnArchName


HIST_BLOCK = 20480   # bytes per query in the workspace's histogram region
HIST_FIRST = 16384   # of which the first-digit histogram, zero between calls


def hist_region(ws_bytes: int) -> int:
    """Bytes of a workspace's histogram region: its first sixteenth, in whole
    per-query blocks."""
    return (ws_bytes // 16) // HIST_BLOCK * HIST_BLOCK


def first_digit_dirty(ws) -> int:
    """Non-zero bytes in the first-digit histograms of every block of the
    workspace's histogram region (which must be zero between calls)."""
    H = hist_region(ws.numel())
    blocks = ws[:H].view(-1, HIST_BLOCK)[:, :HIST_FIRST]
    return int(blocks.count_nonzero())
