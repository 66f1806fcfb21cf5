"""The selection dump (DSA_DUMP_SEL): every line equals the selection the
call returned and the oracle's, also when the fused step is given no
selection buffer; a path that cannot be opened is refused before anything
runs.  (The WASTE page compares selections line by line through such a dump,
section "What is checked".)"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from gpu_common import log
from oracle import oracle as O

pytestmark = pytest.mark.gpu

from deepseek_sparse_attention_amd import binding as B   # noqa: E402
from deepseek_sparse_attention_amd import inputs as I    # noqa: E402


def parse(path):
    out = []
    for line in open(path):
        head, _, toks = line.partition(":")
        f = dict(kv.split("=") for kv in head.split())
        out.append((int(f["q"]), int(f["nvis"]), int(f["count"]), [int(t) for t in toks.split()]))
    return out


def check_dump(lines, nvis, sel_ref, cnt_ref, what):
    assert len(lines) == len(nvis), what
    for j, (q, nv, c, toks) in enumerate(lines):
        assert (q, nv, c) == (j, int(nvis[j]), int(cnt_ref[j])), (what, j)
        assert toks == [int(t) for t in sel_ref[j, :c]], (what, j)


@pytest.mark.parametrize("path", ["fused", "select"])
@pytest.mark.parametrize("give_sel", [True, False])
def test_dump_of_the_fused_step(path, give_sel, tmp_path, monkeypatch):
    monkeypatch.setenv("DSA_ATTN_SEL", "1" if path == "fused" else "0")
    dump = tmp_path / "sel.txt"
    monkeypatch.setenv("DSA_DUMP_SEL", str(dump))
    T = 40000
    w = I.make_workload("dump", 57, I.GEOM_TOKEN, 3, T, np.arange(3), [T, 2051, 30001])
    g = w.geom
    dev = torch.device("cuda")
    t = {k: torch.from_numpy(getattr(w, k)).to(dev) for k in ("cache", "idx_k", "q", "idx_q", "idx_w")}
    sel_ld = g["top_k"] + g["kpool"] - 1
    sel = torch.full((3, sel_ld), -7, dtype=torch.int32, device=dev) if give_sel else None
    cnt = torch.empty(3, dtype=torch.int32, device=dev) if give_sel else None
    out = torch.empty((3, g["n_heads"], g["d_latent"]), dtype=torch.float32, device=dev)
    ws = B.new_workspace(g, 3, T, device=dev)
    b = B.batch(None, torch.from_numpy(w.q_nvis).to(dev), T, 3)
    log(f"dump {path} give_sel={give_sel}")
    B.decode_step(g, b, t["idx_q"], t["idx_w"], t["idx_k"], w.key_rows, t["q"], t["cache"], w.T, sel, sel_ld,
                  cnt, out, None, ws)
    torch.cuda.synchronize()
    rsel, rcnt, _, _ = O.decode_step(g, w.q_seq, w.q_nvis, w.idx_q, w.idx_w, w.idx_k, w.q, w.cache)
    lines = parse(dump)
    check_dump(lines, w.q_nvis, rsel, rcnt, f"{path}/{give_sel}")
    if give_sel:
        s, c = sel.cpu().numpy(), cnt.cpu().numpy()
        for q, _, n, toks in lines:
            assert n == c[q] and toks == s[q, :n].tolist()


def test_dump_of_the_standalone_topk(tmp_path, monkeypatch):
    dump = tmp_path / "topk.txt"
    monkeypatch.setenv("DSA_DUMP_SEL", str(dump))
    g = I.GEOM_KPOOL
    nvis = np.array([9000, 2052, 3], np.int32)
    rows = nvis // g["kpool"]
    rng = np.random.default_rng(8)
    s = rng.integers(-50, 50, (3, int(rows.max()))).astype(np.float32)
    sel_ref, cnt_ref = O.topk(nvis, g["kpool"], g["top_k"], s)
    dev = "cuda"
    b = B.batch(None, torch.from_numpy(nvis).to(dev), int(nvis.max()), 3)
    ws = B.new_workspace(g, 3, int(nvis.max()))
    sel_ld = g["top_k"] + g["kpool"] - 1
    sel = torch.full((3, sel_ld), -9, dtype=torch.int32, device=dev)
    cnt = torch.empty(3, dtype=torch.int32, device=dev)
    B.topk(g, b, torch.from_numpy(s).to(dev), s.shape[1], sel, sel_ld, cnt, ws)
    torch.cuda.synchronize()
    check_dump(parse(dump), nvis, sel_ref, cnt_ref, "topk")


def test_unwritable_dump_path_is_refused(tmp_path, monkeypatch):
    monkeypatch.setenv("DSA_DUMP_SEL", str(tmp_path / "no_such_dir" / "sel.txt"))
    g = I.GEOM_TOKEN
    nvis = np.array([5000], np.int32)
    s = np.zeros((1, 5000), np.float32)
    dev = "cuda"
    b = B.batch(None, torch.from_numpy(nvis).to(dev), 5000, 1)
    ws = B.new_workspace(g, 1, 5000)
    sel = torch.full((1, 2048), -9, dtype=torch.int32, device=dev)
    cnt = torch.full((1,), -9, dtype=torch.int32, device=dev)
    with pytest.raises(B.DSAError) as e:
        B.topk(g, b, torch.from_numpy(s).to(dev), 5000, sel, 2048, cnt, ws)
    assert e.value.status == B.DSA_ERR_ARG
    torch.cuda.synchronize()
    assert bool((sel == -9).all()) and int(cnt[0]) == -9
    assert not os.path.exists(tmp_path / "no_such_dir")
