"""Randomised parity of the fused step with the oracle: batches drawn from a
seeded generator, each with its own geometry (token or k-pool, with or
without RoPE columns), top_k, sequence count, context lengths, query map
(some as runs of consecutive positions, the prefill shape) and key range
(narrow ranges make ties).  Selections must equal the oracle's bit for bit,
attention must be within the tolerance."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import check_attention, check_selection, log, oracle_decode, gpu_arch

pytestmark = pytest.mark.gpu

from deepseek_sparse_attention_amd import binding as B            # noqa: E402
from deepseek_sparse_attention_amd import inputs as I             # noqa: E402
from deepseek_sparse_attention_amd.workload import DeviceWorkload  # noqa: E402

N_CASES = 24


def setup_module():
    assert gpu_arch().startswith("gfx950")
    B.device_check()


def draw(i: int):
    rng = np.random.default_rng(9000 + i)
    kpool = int(rng.choice([1, 4]))
    d_rope = int(rng.choice([0, 64]))
    top_k = int(rng.choice([16, 64, 256, 2048, 4096]))
    g = dict(I.GEOM_TOKEN, kpool=kpool, d_rope=d_rope, top_k=top_k)
    n_seq = int(rng.integers(1, 5))
    T = int(rng.integers(1, 24001))
    if rng.random() < 0.3:
        # a run of consecutive positions per sequence (prefill / verify shape)
        run = int(rng.integers(2, 10))
        q_seq, q_nvis = [], []
        for s in range(n_seq):
            last = int(rng.integers(run, T + 1)) if T >= run else run
            last = min(last, T)
            for j in range(run):
                q_seq.append(s)
                q_nvis.append(max(1, last - run + 1 + j))
    else:
        n_q = int(rng.integers(1, 9))
        q_seq = rng.integers(0, n_seq, n_q).tolist()
        q_nvis = rng.integers(1, T + 1, n_q).tolist()
        if rng.random() < 0.5:
            q_nvis[0] = T
    key_range = [(-8, 8), (-2, 2), (-1, 1)][int(rng.integers(0, 3))]
    return g, n_seq, T, q_seq, q_nvis, key_range


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_batch_matches_oracle(i):
    g, n_seq, T, q_seq, q_nvis, kr = draw(i)
    name = f"random{i}"
    log(f"{name}: kpool {g['kpool']} d_rope {g['d_rope']} top_k {g['top_k']} n_seq {n_seq} T {T} "
        f"n_q {len(q_seq)} keys {kr}")
    w = I.make_workload(name, 400 + i, g, n_seq, T, q_seq, q_nvis, key_range=kr)
    dw = DeviceWorkload(w)
    dw.sel.fill_(-7)
    dw.decode_step()
    torch.cuda.synchronize()
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, name)
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, name)
