"""GPU parity of the k-pool key producer (dsa_pool_append) against the CPU
oracle, and the k-pool decode step fed with the pool keys it produces."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import log, check_attention, gpu_arch
from oracle import oracle as O
from deepseek_sparse_attention_amd import binding as B
from deepseek_sparse_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

DI = 128
SENT = 0x7F7F


def setup_module():
    assert gpu_arch().startswith("gfx950"), gpu_arch()


def _cells(rng, n_seq, n):
    keys = I.f32_to_bf16_bits((rng.standard_normal((n_seq, n, DI)) * 3).astype(np.float32))
    gates = I.f32_to_bf16_bits((rng.standard_normal((n_seq, n, DI)) * 2).astype(np.float32))
    return np.concatenate([keys, gates], axis=-1)


def _pos_emb(rng):
    return rng.standard_normal((4, DI)).astype(np.float32)


def _ulps(a, b):
    """Distance in bf16 units of two arrays of bf16 bits (same-sign values)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))


def _key_bound(cells, pools):
    """[len(pools), DI]: largest |key| among each pool's four tokens; the fp32
    evaluation of a pool key is within 2^-20 of that (a 4-term weighted mean)."""
    keys = np.abs(I.bf16_bits_to_f32(cells[..., :DI]).astype(np.float64))
    return np.stack([keys[4 * p:4 * p + 4].max(0) for p in pools])


def _check_keys(got, ref, what, keymax):
    """Each pool key within 1 bf16 ulp of the oracle's, or, where the key is
    small against its terms (cancellation), within the fp32 evaluation error
    2^-20 * max |key_j| plus 1 ulp; at least 99% bit-equal."""
    d = _ulps(got, ref)
    g = I.bf16_bits_to_f32(got).astype(np.float64)
    r = I.bf16_bits_to_f32(ref).astype(np.float64)
    ulp = np.abs(r) * 2.0 ** -7 + 1e-38
    ok = (d <= 1) | (np.abs(g - r) <= 2.0 ** -20 * keymax + ulp)
    exact = float((d == 0).mean())
    log(f"{what}: {got.size} values, {100 * exact:.3f}% bit-equal, max {int(d.max())} ulp "
        f"({int((d > 1).sum())} beyond 1 ulp, all near cancellation: {bool(ok.all())})")
    assert ok.all(), f"{what}: pool key outside its bound"
    assert exact >= 0.99, f"{what}: only {100 * exact:.2f}% bit-equal"


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.to("cuda")


def _host_u16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _check_rolling(got, ref, end, what):
    """Slots 0 .. end mod 4 - 1 hold the incomplete pool; the rest are unspecified."""
    for s in range(len(end)):
        k = int(end[s]) % 4
        assert np.array_equal(got[s, :k], ref[s, :k]), f"{what}: rolling buffer of sequence {s}"


def _pack_new(cells, n_tok, n_new):
    stride = max(1, int(np.max(n_new)))
    out = np.zeros((cells.shape[0], stride, 2 * DI), np.uint16)
    for s in range(cells.shape[0]):
        out[s, :n_new[s]] = cells[s, n_tok[s]:n_tok[s] + n_new[s]]
    return out


def test_pool_append_matches_oracle():
    """One chunked append per sequence from every partial-pool state: the
    pools it completes within 1 ulp of the oracle (99% bit-equal), the
    rolling buffer bit-exact, every other pool untouched."""
    log("pool append chunk")
    rng = np.random.default_rng(5)
    n_tok = np.array([0, 1, 2, 3, 7, 10, 5], np.int32)
    n_new = np.array([1, 3, 4, 9, 13, 0, 400], np.int32)
    total = n_tok + n_new
    cells = _cells(rng, 7, int(total.max()))
    pos = _pos_emb(rng)
    P = int(total.max()) // 4 + 2
    roll = np.zeros((7, 4, 2 * DI), np.uint16)
    pk = np.full((7, P, DI), SENT, np.uint16)
    O.pool_append(np.zeros(7, np.int32), n_tok, _pack_new(cells, np.zeros(7, np.int32), n_tok), roll, pk, pos)
    new = _pack_new(cells, n_tok, n_new)
    d_roll, d_pk = _dev(roll), _dev(pk)
    B.pool_append(_dev(n_tok), _dev(n_new), int(n_new.max()), _dev(new), d_roll, d_pk, _dev(pos))
    O.pool_append(n_tok, n_new, new, roll, pk, pos)
    torch.cuda.synchronize()
    g_roll, g_pk = _host_u16(d_roll), _host_u16(d_pk)
    _check_rolling(g_roll, roll, total, "chunk")
    fresh = np.zeros(pk.shape[:2], bool)
    for s in range(7):
        fresh[s, n_tok[s] // 4:total[s] // 4] = True
    assert np.array_equal(g_pk[~fresh], pk[~fresh]), "a pool the call does not complete was written"
    km = np.zeros(pk.shape)
    for s_ in range(7):
        ps = list(range(n_tok[s_] // 4, total[s_] // 4))
        if ps:
            km[s_, ps] = _key_bound(cells[s_], ps)
    _check_keys(g_pk[fresh], pk[fresh], "chunk", km[fresh])


def test_pool_append_decode_loop():
    """Twenty-one single-token steps on sequences that start at lengths 0..5."""
    log("pool append decode loop")
    rng = np.random.default_rng(6)
    n_seq, steps = 6, 21
    start = np.arange(n_seq, dtype=np.int32)
    cells = _cells(rng, n_seq, int(start.max()) + steps)
    pos = _pos_emb(rng)
    P = (int(start.max()) + steps) // 4 + 1
    roll = np.zeros((n_seq, 4, 2 * DI), np.uint16)
    pk = np.full((n_seq, P, DI), SENT, np.uint16)
    O.pool_append(np.zeros(n_seq, np.int32), start, _pack_new(cells, np.zeros(n_seq, np.int32), start), roll, pk, pos)
    d_roll, d_pk, d_pos = _dev(roll), _dev(pk), _dev(pos)
    ones = np.ones(n_seq, np.int32)
    d_ones = _dev(ones)
    for i in range(steps):
        n_tok = start + i
        new = _pack_new(cells, n_tok, ones)
        B.pool_append(_dev(n_tok), d_ones, 1, _dev(new), d_roll, d_pk, d_pos)
        O.pool_append(n_tok, ones, new, roll, pk, pos)
    torch.cuda.synchronize()
    _check_rolling(_host_u16(d_roll), roll, start + steps, "decode loop")
    g = _host_u16(d_pk)
    done = np.zeros(pk.shape[:2], bool)
    for s in range(n_seq):
        done[s, start[s] // 4:(start[s] + steps) // 4] = True
    assert np.array_equal(g[~done], pk[~done])
    km = np.zeros(pk.shape)
    for s_ in range(n_seq):
        ps = list(range(start[s_] // 4, (start[s_] + steps) // 4))
        km[s_, ps] = _key_bound(cells[s_], ps)
    _check_keys(g[done], pk[done], "decode loop", km[done])


def test_pool_append_guards():
    """Sequences with n_new > max_new or negative counts are left untouched,
    and pools at or past pool_stride are not written."""
    log("pool append guards")
    rng = np.random.default_rng(7)
    cells = _cells(rng, 4, 40)
    pos = _pos_emb(rng)
    n_tok = np.array([0, -1, 0, 0], np.int32)
    n_new = np.array([40, 4, 9, -2], np.int32)
    roll = np.full((4, 4, 2 * DI), 0x1234, np.uint16)
    pk = np.full((4, 6, DI), SENT, np.uint16)              # only 6 pools fit
    d_roll, d_pk = _dev(roll), _dev(pk)
    new = np.ascontiguousarray(cells[:, :40])
    B.pool_append(_dev(n_tok), _dev(n_new), 8, _dev(new), d_roll, d_pk, _dev(pos))   # max_new 8 < 40, 9
    torch.cuda.synchronize()
    assert np.array_equal(_host_u16(d_roll), roll) and np.array_equal(_host_u16(d_pk), pk)
    n_new = np.array([40, 0, 0, 0], np.int32)
    B.pool_append(_dev(n_tok * 0), _dev(n_new), 40, _dev(new), d_roll, d_pk, _dev(pos))
    torch.cuda.synchronize()
    ref_roll = roll.copy()
    ref_pk = np.full((4, 10, DI), SENT, np.uint16)
    O.pool_append(np.zeros(4, np.int32), n_new, new, ref_roll, ref_pk, pos)
    g_pk = _host_u16(d_pk)
    _check_keys(g_pk[0], ref_pk[0, :6], "first 6 pools", _key_bound(cells[0], range(6)))
    assert np.array_equal(g_pk[1:], pk[1:])
    _check_rolling(_host_u16(d_roll)[:1], ref_roll[:1], [40], "first sequence")


def test_kpool_step_on_produced_pool_keys():
    """End to end for the k-pool variant: the producer builds the pool keys
    of a 16,387-token sequence from its cells, and the fused step selects and
    attends on them.  The keys are not integers, so scores are checked
    against an fp32 accumulation bound, selections may differ only at rows
    whose score lies within twice that bound of the threshold, and the
    attention is checked on the GPU's own selection."""
    log("k-pool step on produced keys")
    rng = np.random.default_rng(8)
    T = 16387
    geom = dict(I.GEOM_KPOOL)
    cells = _cells(rng, 1, T)
    pos = _pos_emb(rng)
    P = T // 4
    d_roll = torch.zeros((1, 4, 2 * DI), dtype=torch.int16, device="cuda")
    d_pk = torch.zeros((1, P, DI), dtype=torch.int16, device="cuda")
    B.pool_append(_dev(np.zeros(1, np.int32)), _dev(np.array([T], np.int32)), T, _dev(cells), d_roll, d_pk, _dev(pos))
    roll = np.zeros((1, 4, 2 * DI), np.uint16)
    pk = np.zeros((1, P, DI), np.uint16)
    O.pool_append(np.zeros(1, np.int32), np.array([T], np.int32), cells, roll, pk, pos)
    torch.cuda.synchronize()
    keys = _host_u16(d_pk)
    _check_keys(keys, pk, "sequence", _key_bound(cells[0], range(P))[None])

    n_q = 3
    nvis = np.array([T, T - 1, T - 4000], np.int32)
    q_seq = np.zeros(n_q, np.int32)
    qi = I.f32_to_bf16_bits(rng.integers(-8, 9, size=(n_q, 32, DI)).astype(np.float32))
    w = rng.integers(1, 5, size=(n_q, 32)).astype(np.float32)
    q = I.f32_to_bf16_bits(rng.standard_normal((n_q, 64, 512)).astype(np.float32))
    cache = I.f32_to_bf16_bits(rng.standard_normal((1, T, 512)).astype(np.float32))
    ref_s = O.index_scores(q_seq, nvis, 4, qi, w, keys)
    dev = "cuda"
    b = B.batch(torch.from_numpy(q_seq).to(dev), torch.from_numpy(nvis).to(dev), T, 1)
    ws = B.new_workspace(geom, n_q, T)
    sel_ld = geom["top_k"] + 3
    ld = P + 1
    scores = torch.full((n_q, ld), float("nan"), device=dev)
    d_keys = _dev(keys)
    B.index_scores(geom, b, _dev(qi), _dev(w), d_keys, P, scores, ld)
    sel = torch.full((n_q, sel_ld), -9, dtype=torch.int32, device=dev)
    cnt = torch.zeros(n_q, dtype=torch.int32, device=dev)
    out = torch.empty((n_q, 64, 512), device=dev)
    lse = torch.empty((n_q, 64), device=dev)
    B.decode_step(geom, b, _dev(qi), _dev(w), d_keys, P, _dev(q), _dev(cache), T, sel, sel_ld, cnt, out, lse, ws)
    torch.cuda.synchronize()
    got_s = scores.cpu().numpy()
    sel_g, cnt_g = sel.cpu().numpy(), cnt.cpu().numpy()
    kf = I.bf16_bits_to_f32(keys[0]).astype(np.float64)
    qf = I.bf16_bits_to_f32(qi).astype(np.float64)
    keep = geom["top_k"] // 4
    for j in range(n_q):
        rows = int(nvis[j]) // 4
        # |fp32 result - exact| <= 2^-20 * sum_h w_h sum_d |q_hd k_rd| (128-term sums, exact products)
        bound = 2.0 ** -20 * (np.abs(kf[:rows]) @ np.abs(qf[j]).T) @ w[j].astype(np.float64)
        err = np.abs(got_s[j, :rows].astype(np.float64) - ref_s[j, :rows].astype(np.float64))
        assert (err <= bound).all(), f"query {j}: score error {err.max():.3e} over its bound"
        order = np.lexsort((np.arange(rows), -ref_s[j, :rows].astype(np.float64)))
        thr = float(ref_s[j, order[keep - 1]])
        want = set(order[:keep].tolist())
        have = set((sel_g[j, :keep * 4:4] // 4).tolist())
        assert cnt_g[j] == keep * 4 + int(nvis[j]) % 4
        for p in want ^ have:
            assert abs(float(ref_s[j, p]) - thr) <= 2 * bound[p], f"query {j}: pool {p} differs away from a tie"
        log(f"query {j}: {len(want ^ have) // 2} near-tie swaps, max score error {err.max():.2e}")
    out_ref, lse_ref = O.mla_attend(q_seq, 512, 0, 1 / 16, q, cache, sel_g, cnt_g)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), out_ref, lse_ref, "k-pool on produced keys")
