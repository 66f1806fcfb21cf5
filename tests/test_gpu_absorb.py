"""GPU parity of the absorption GEMMs (dsa_absorb_query, dsa_project_output)
against the CPU oracle, and of the absorbed decode step end to end."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import log, gpu_arch, row_rel_err, ATTN_TOL
from oracle import oracle as O
from deepseek_sparse_attention_amd import binding as B
from deepseek_sparse_attention_amd import inputs as I
from deepseek_sparse_attention_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu


def setup_module():
    assert gpu_arch().startswith("gfx950"), gpu_arch()


def _bf(x):
    return I.f32_to_bf16_bits(np.asarray(x, np.float32))


def _f(b):
    return I.bf16_bits_to_f32(b).astype(np.float64)


def _dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _host16(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n_q", [1, 8, 37, 130, 300])
@pytest.mark.parametrize("d_rope", [64, 0])
def test_absorb_matches_oracle(n_q, d_rope):
    """q_abs within 1 bf16 ulp of the oracle, or within the fp32 accumulation
    bound 2^-16 sum_k |q_k W_kn| plus 1 ulp; at least 99% bit-equal; the RoPE
    part copied exactly."""
    log(f"absorb n_q={n_q} d_rope={d_rope}")
    rng = np.random.default_rng(100 + n_q + d_rope)
    qn = _bf(rng.standard_normal((n_q, 64, 256)))
    qr = _bf(rng.standard_normal((n_q, 64, d_rope))) if d_rope else None
    W = _bf(rng.standard_normal((64, 256, 512)) * 0.05)
    ref = O.absorb_query(qn, qr, W)
    out = torch.full((n_q, 64, 512 + d_rope), 0x7F7F, dtype=torch.int16, device="cuda")
    B.absorb_query(_dev16(qn), _dev16(qr) if d_rope else None, _dev16(W), out)
    torch.cuda.synchronize()
    got = _host16(out)
    if d_rope:
        assert np.array_equal(got[:, :, 512:], ref[:, :, 512:]), "RoPE part"
    g, r = _f(got[:, :, :512]), _f(ref[:, :, :512])
    absum = np.einsum("mhk,hkn->mhn", np.abs(_f(qn)), np.abs(_f(W)))
    ok = (g == r) | (np.abs(g - r) <= 2.0 ** -16 * absum + np.abs(r) * 2.0 ** -7)
    exact = float((got[:, :, :512] == ref[:, :, :512]).mean())
    log(f"absorb: {100 * exact:.3f}% bit-equal, max |diff| {np.abs(g - r).max():.3e}")
    assert ok.all() and exact >= 0.99


@pytest.mark.parametrize("n_q", [1, 8, 37, 130, 300])
def test_project_matches_oracle(n_q):
    """ctx within 2^-14 sum_j |o_j W_ij| of the oracle (o as bf16 hi + lo)."""
    log(f"project n_q={n_q}")
    rng = np.random.default_rng(200 + n_q)
    o = rng.standard_normal((n_q, 64, 512)).astype(np.float32)
    W = _bf(rng.standard_normal((64, 256, 512)) * 0.05)
    ref = O.project_output(o, W)
    ctx = torch.full((n_q, 64, 256), float("nan"), device="cuda")
    B.project_output(torch.from_numpy(o).cuda(), _dev16(W), ctx)
    torch.cuda.synchronize()
    got = ctx.cpu().numpy().astype(np.float64)
    bound = 2.0 ** -14 * np.einsum("mhj,hij->mhi", np.abs(o).astype(np.float64), np.abs(_f(W)))
    err = np.abs(got - ref)
    log(f"project: max |diff| {err.max():.3e}, max diff/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()


def test_absorbed_decode_step_end_to_end():
    """Absorb -> fused step -> project on the GPU against the same chain in
    the oracle: selections bit-exact (the indexer does not see q), outputs
    within the attention tolerance relative to each row."""
    log("absorbed step end to end")
    w = I.config("c0")
    rng = np.random.default_rng(300)
    n_q = w.n_q
    qn = _bf(rng.standard_normal((n_q, 64, 256)) * 0.5)
    qr = w.q[:, :, 512:].copy()
    Wk = _bf(rng.standard_normal((64, 256, 512)) * 0.05)
    Wv = _bf(rng.standard_normal((64, 256, 512)) * 0.05)
    dw = DeviceWorkload(w)
    B.absorb_query(_dev16(qn), _dev16(qr), _dev16(Wk), dw.q.view(torch.int16))
    dw.decode_step()
    ctx = torch.empty((n_q, 64, 256), device="cuda")
    B.project_output(dw.out, _dev16(Wv), ctx)
    torch.cuda.synchronize()
    q_abs = O.absorb_query(qn, qr, Wk)
    sel, cnt, out, lse = O.decode_step(w.geom, w.q_seq, w.q_nvis, w.idx_q, w.idx_w, w.idx_k, q_abs, w.cache)
    ref = O.project_output(out, Wv)
    assert np.array_equal(dw.sel.cpu().numpy(), sel) and np.array_equal(dw.sel_count.cpu().numpy(), cnt)
    err = row_rel_err(ctx.cpu().numpy(), ref)
    log(f"absorbed step: ctx row-rel err {err:.3e}")
    assert err <= ATTN_TOL


def test_absorption_query_count_bounds():
    """n_q below 1 or above 2^20 is refused before any launch (the 1-D grid of
    512 work-groups per 64 queries must stay under 2^32 work-items)."""
    log("absorption n_q bounds")
    buf = torch.zeros(1 << 16, dtype=torch.int16, device="cuda")
    p = buf.data_ptr()
    for n_q, want in ((0, B.DSA_ERR_ARG), ((1 << 20) + 1, B.DSA_ERR_UNSUPPORTED)):
        assert B._lib.dsa_absorb_query(n_q, 0, p, None, p, p, None) == want
        assert B._lib.dsa_project_output(n_q, p, p, p, None) == want
