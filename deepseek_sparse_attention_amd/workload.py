"""Device-resident copy of a synthetic workload and one call of the fused
step on it.  Plumbing only: torch allocates and uploads, the C ABI computes.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from .inputs import Workload


def run_hint(q_seq) -> int:
    """Length of the runs of consecutive queries that share a sequence, if
    every run has the same length >= 2, else 0 (no hint)."""
    q_seq = np.asarray(q_seq)
    if q_seq.size < 2:
        return 0
    cut = np.flatnonzero(np.diff(q_seq) != 0) + 1
    lengths = np.diff(np.concatenate(([0], cut, [q_seq.size])))
    return int(lengths[0]) if lengths[0] >= 2 and (lengths == lengths[0]).all() else 0


class DeviceWorkload:
    """Uploads a host ``Workload`` and owns outputs and a workspace for it."""

    def __init__(self, w: Workload, device: str = "cuda", sel_ld: int | None = None, seq_map: str = "auto"):
        """seq_map "auto": when query i reads sequence i, the batch passes a
        NULL q_seq (the C ABI's convention for that case, which lets the
        scorer request its first keys before the query's fields arrive);
        "always": the device array in every case."""
        self.w = w
        self.geom = w.geom
        dev = torch.device(device)

        def up(a):
            return torch.from_numpy(a).to(dev)

        self.cache = up(w.cache)
        self.idx_k = up(w.idx_k)
        self.q = up(w.q)
        self.idx_q = up(w.idx_q)
        self.idx_w = up(w.idx_w)
        self.q_seq = up(w.q_seq)
        self.q_nvis = up(w.q_nvis)
        self.max_nvis = int(w.q_nvis.max())
        self.n_q = w.n_q
        self.sel_ld = sel_ld or (self.geom["top_k"] + self.geom["kpool"] - 1)
        self.sel = torch.empty((self.n_q, self.sel_ld), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty(self.n_q, dtype=torch.int32, device=dev)
        self.out = torch.empty((self.n_q, self.geom["n_heads"], self.geom["d_latent"]), dtype=torch.float32,
                               device=dev)
        self.lse = torch.empty((self.n_q, self.geom["n_heads"]), dtype=torch.float32, device=dev)
        self.ws = B.new_workspace(self.geom, self.n_q, self.max_nvis, device=dev)
        identity = w.n_q <= w.n_seq and np.array_equal(w.q_seq, np.arange(w.n_q))
        self.batch = B.batch(None if (identity and seq_map == "auto") else self.q_seq, self.q_nvis, self.max_nvis,
                             w.n_seq, run_hint(w.q_seq))

    def decode_step(self, stream=None, with_sel: bool = True) -> None:
        B.decode_step(self.geom, self.batch, self.idx_q, self.idx_w, self.idx_k, self.w.key_rows, self.q,
                      self.cache, self.w.T, self.sel if with_sel else None, self.sel_ld,
                      self.sel_count if with_sel else None, self.out, self.lse, self.ws, stream)
