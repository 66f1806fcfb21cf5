"""GPU parity of the indexer input preparation (dsa_index_prepare: rope,
Walsh-Hadamard rotation, rounding to bf16 or f16, key-cache append) against
the CPU oracle; f16 indexer scoring bit-exact on integer inputs; and the
prepared inputs through the fused step end to end."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import log, gpu_arch, check_attention, check_selection, oracle_decode
from oracle import oracle as O
from deepseek_sparse_attention_amd import binding as B
from deepseek_sparse_attention_amd import inputs as I
from deepseek_sparse_attention_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu

DI, HI = 128, 32
SENTINEL = 0x1357


def setup_module():
    assert gpu_arch().startswith("gfx950"), gpu_arch()


def _geom(f16):
    return dict(I.GEOM_TOKEN, idx_f16=int(f16))


def _decode16(bits, f16):
    if f16:
        return bits.view(np.float16).astype(np.float64)
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def _ulp16(v, f16):
    """Spacing of the 16-bit format at |v| (bf16: 8 significant bits; f16: 11,
    subnormal below 2^-14)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-300)))
    if f16:
        return 2.0 ** (np.maximum(e, -14) - 10)
    return 2.0 ** (e - 7)


def _check_prepared(got, x, pos, f16, what):
    """got: uint16 [n, 128] prepared vectors; x: float32 [n, 128] inputs at
    positions pos [n].  Each element must be the oracle's rounding of the
    exact transform, or lie within half a unit in the last place plus the fp32
    evaluation bound 2^-20 sum_k |x_k| / sqrt(128) of the exact value; at least
    99% of the elements must be bit-equal to the oracle's."""
    exact = np.stack([O.index_rotate(x[i].astype(np.float64), int(pos[i]), 64) for i in range(x.shape[0])])
    ref = O.round16(exact, f16)
    g = _decode16(got, f16)
    bound = 0.5 * _ulp16(g, f16) + 2.0 ** -20 * np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True) / np.sqrt(DI)
    ok = (got == ref) | (np.abs(g - exact) <= bound)
    same = float((got == ref).mean())
    log(f"{what}: {100 * same:.3f}% bit-equal to the oracle, {int((~ok).sum())} outside the bound")
    assert ok.all(), f"{what}: {int((~ok).sum())} elements outside the bound"
    assert same >= 0.99, f"{what}: only {100 * same:.2f}% bit-equal"


@pytest.mark.parametrize("f16", [False, True], ids=["bf16", "f16"])
@pytest.mark.parametrize("n_q,n_new,keyed", [(1, 1, True), (8, 8, False), (37, 513, True)])
def test_prepare_matches_oracle(f16, n_q, n_new, keyed):
    """Queries at positions up to 2^21 and keys at random rows of three
    sequences: every prepared vector meets the bar, the keys land on their
    rows and no other row of the cache changes."""
    log(f"prepare f16={f16} n_q={n_q} n_new={n_new} keyed={keyed}")
    rng = np.random.default_rng(200 + n_q + n_new + int(f16))
    n_seq = 3 if keyed else max(n_new, 1)
    stride = 1 << 15
    q_in, k_in = I.indexer_projections(int(rng.integers(1 << 30)), n_q, n_new)
    q_nvis = rng.integers(1, 1 << 21, n_q).astype(np.int32)
    q_nvis[0] = 1
    if keyed:
        flat = rng.choice(n_seq * stride, n_new, replace=False)
        flat[-1] = n_seq * stride - 1
        k_seq, k_pos = (flat // stride).astype(np.int32), (flat % stride).astype(np.int32)
    else:
        k_seq, k_pos = None, rng.integers(0, stride, n_new).astype(np.int32)
    g = _geom(f16)
    dev = "cuda"
    b = B.batch(torch.zeros(n_q, dtype=torch.int32, device=dev), torch.from_numpy(q_nvis).to(dev),
                int(q_nvis.max()), n_seq)
    q_out = torch.full((n_q, HI, DI), SENTINEL, dtype=torch.int16, device=dev)
    cache = torch.full((n_seq, stride, DI), SENTINEL, dtype=torch.int16, device=dev)
    B.index_prepare(g, b, torch.from_numpy(q_in).to(dev), q_out,
                    None if k_seq is None else torch.from_numpy(k_seq).to(dev), torch.from_numpy(k_pos).to(dev),
                    torch.from_numpy(k_in).to(dev), cache, stride)
    torch.cuda.synchronize()
    got_q = q_out.cpu().numpy().view(np.uint16).reshape(n_q * HI, DI)
    _check_prepared(got_q, q_in.reshape(n_q * HI, DI), np.repeat(q_nvis.astype(np.int64) - 1, HI), f16, "queries")
    ref_q, _ = O.index_prepare(q_nvis, q_in, None, np.zeros(0, np.int32), np.zeros((0, DI), np.float32),
                               np.zeros((1, 1, DI), np.uint16), 64, f16)
    assert float((got_q == ref_q.reshape(n_q * HI, DI)).mean()) >= 0.99, "query positions differ from the oracle's"
    seqs = np.arange(n_new) if k_seq is None else k_seq
    touched = (cache != SENTINEL).any(dim=2).nonzero().cpu().numpy()
    want = sorted(zip(seqs.tolist(), k_pos.tolist()))
    assert sorted(map(tuple, touched.tolist())) == want, "rows written differ from the keys' rows"
    got_k = cache[torch.from_numpy(seqs.astype(np.int64)).to(dev), torch.from_numpy(k_pos.astype(np.int64)).to(dev)]
    _check_prepared(got_k.cpu().numpy().view(np.uint16), k_in, k_pos, f16, "keys")


@pytest.mark.parametrize("f16", [False, True], ids=["bf16", "f16"])
def test_prepare_guards(f16):
    """Keys aimed outside [0, n_seq) x [0, key_seq_stride) are not written and
    nothing else changes; host-side refusals enqueue nothing."""
    log(f"prepare guards f16={f16}")
    dev = "cuda"
    n_seq, stride = 2, 64
    g = _geom(f16)
    q_in, k_in = I.indexer_projections(9, 1, 6)
    k_seq = np.array([0, 1, -1, 2, 0, 1], np.int32)
    k_pos = np.array([3, 63, 5, 0, 64, -1], np.int32)
    b = B.batch(torch.zeros(1, dtype=torch.int32, device=dev), torch.tensor([17], dtype=torch.int32, device=dev),
                17, n_seq)
    cache = torch.full((n_seq, stride, DI), SENTINEL, dtype=torch.int16, device=dev)
    q_out = torch.full((1, HI, DI), SENTINEL, dtype=torch.int16, device=dev)
    args = (torch.from_numpy(q_in).to(dev), q_out, torch.from_numpy(k_seq).to(dev), torch.from_numpy(k_pos).to(dev),
            torch.from_numpy(k_in).to(dev), cache, stride)
    B.index_prepare(g, b, *args)
    torch.cuda.synchronize()
    touched = sorted(map(tuple, (cache != SENTINEL).any(dim=2).nonzero().cpu().numpy().tolist()))
    assert touched == [(0, 3), (1, 63)], touched
    _check_prepared(cache[0, 3:4].cpu().numpy().view(np.uint16), k_in[:1], k_pos[:1], f16, "guarded key 0")
    _check_prepared(cache[1, 63:64].cpu().numpy().view(np.uint16), k_in[1:2], k_pos[1:2], f16, "guarded key 1")
    before = (cache.clone(), q_out.clone())
    refusals = [
        (dict(I.GEOM_KPOOL, idx_f16=0), b, args, 8.0e6, B.DSA_ERR_UNSUPPORTED),
        (g, b, args, 1.0, B.DSA_ERR_ARG),
        (g, b, (args[0], None) + args[2:], 8.0e6, B.DSA_ERR_ARG),
        (g, b, (args[0], args[1], None) + args[3:], 8.0e6, B.DSA_ERR_ARG),   # 6 keys, 2 sequences, no k_seq
    ]
    for gg, bb, aa, base, status in refusals:
        with pytest.raises(B.DSAError) as e:
            B.index_prepare(gg, bb, *aa, rope_base=base)
        assert e.value.status == status, e.value
    torch.cuda.synchronize()
    assert torch.equal(cache, before[0]) and torch.equal(q_out, before[1])


def _as_f16(w):
    """The same integer-valued workload with its indexer inputs as f16 bits."""
    def conv(bits):
        return I.bf16_bits_to_f32(bits).astype(np.float16).view(np.uint16)
    w.idx_q = conv(w.idx_q)
    w.idx_k = conv(w.idx_k)
    w.geom = dict(w.geom, idx_f16=1)
    return w


F16_CASES = [
    ("tok_mixed", 2, 5003, [0, 1, 1, 0], [5003, 4097, 1500, 2049]),
    ("tok_prefill", 1, 4096, [0] * 24, list(range(4073, 4097))),
    ("tok_window", 2, 9000, [0, 0, 0, 1, 1, 1], [8998, 8999, 9000, 7000, 7001, 7002]),
    # long contexts, whose decode scorer runs 8-wave work-groups: 1,024-row
    # tiles for one query, 2,048 for three, 4,096 for five
    ("tok_long1", 1, 131072, [0], [131072]),
    ("tok_long3", 3, 131072, [0, 1, 2], [131072, 131000, 100003]),
    ("tok_long5", 5, 131072, [0, 1, 2, 3, 4], [131072, 131071, 90000, 131072, 70001]),
]


@pytest.mark.parametrize("case", list(enumerate(F16_CASES)), ids=[c[0] for c in F16_CASES])
def test_f16_scores_and_step_bit_exact(case):
    """Integer-valued indexer inputs are exact in f16 as in bf16: the f16
    scorer (decode, verify-window and prefill layouts) gives the oracle's
    scores bit for bit, and the fused step its selections."""
    i, (name, n_seq, T, q_seq, q_nvis) = case
    log(f"f16 scores {name}")
    w = _as_f16(I.make_workload(name, 300 + i, I.GEOM_TOKEN, n_seq, T, q_seq, q_nvis))
    dw = DeviceWorkload(w)
    ld = dw.max_nvis + 3
    scores = torch.full((w.n_q, ld), float("nan"), device="cuda")
    B.index_scores(w.geom, dw.batch, dw.idx_q, dw.idx_w, dw.idx_k, w.key_rows, scores, ld)
    dw.decode_step()
    torch.cuda.synchronize()
    ref = O.index_scores(w.q_seq, w.q_nvis, 1, w.idx_q, w.idx_w, w.idx_k, score_ld=ld, f16=True)
    got = scores.cpu().numpy()
    for j in range(w.n_q):
        rows = int(w.q_nvis[j])
        assert np.array_equal(got[j, :rows], ref[j, :rows]), f"{name} q{j}"
    sel, cnt, out, lse = oracle_decode(w)
    check_selection(dw.sel.cpu().numpy(), dw.sel_count.cpu().numpy(), sel, cnt, name)
    check_attention(dw.out.cpu().numpy(), dw.lse.cpu().numpy(), out, lse, name)


@pytest.mark.parametrize("f16", [False, True], ids=["bf16", "f16"])
def test_prepared_step_end_to_end(f16):
    """Float projections of two 12,000-token sequences are prepared on the
    GPU (keys appended at their positions, queries at n_vis - 1) and the
    fused step runs on them.  The prepared vectors meet the preparation bar;
    the GPU scores lie within the fp32 accumulation bound
    2^-20 sum_h w_h sum_d |q_hd k_rd| of the oracle's scores on the same
    prepared inputs; a selection may differ from the oracle's only at rows
    whose score lies within twice that bound of the k-th score; attention is
    checked on the GPU's own selection."""
    log(f"prepared step f16={f16}")
    dev = "cuda"
    g = _geom(f16)
    T, n_seq = 12000, 2
    q_seq = np.array([0, 0, 1], np.int32)
    q_nvis = np.array([T, T - 777, T - 5], np.int32)
    n_q = q_seq.size
    q_in, k_in = I.indexer_projections(77 + int(f16), n_q, n_seq * T)
    k_seq = np.repeat(np.arange(n_seq, dtype=np.int32), T)
    k_pos = np.tile(np.arange(T, dtype=np.int32), n_seq)
    rng = np.random.default_rng(78)
    w_idx = (rng.random((n_q, HI)) + 0.5).astype(np.float32)
    q = I.f32_to_bf16_bits(rng.standard_normal((n_q, 64, 576)).astype(np.float32))
    cache = I.f32_to_bf16_bits(rng.standard_normal((n_seq, T, 576)).astype(np.float32))
    b = B.batch(torch.from_numpy(q_seq).to(dev), torch.from_numpy(q_nvis).to(dev), T, n_seq)
    d_qi = torch.empty((n_q, HI, DI), dtype=torch.int16, device=dev)
    d_k = torch.full((n_seq, T, DI), SENTINEL, dtype=torch.int16, device=dev)
    B.index_prepare(g, b, torch.from_numpy(q_in).to(dev), d_qi, torch.from_numpy(k_seq).to(dev),
                    torch.from_numpy(k_pos).to(dev), torch.from_numpy(k_in).to(dev), d_k, T)
    ws = B.new_workspace(g, n_q, T)
    sel_ld = g["top_k"]
    scores = torch.full((n_q, T), float("nan"), device=dev)
    d_w = torch.from_numpy(w_idx).to(dev)
    B.index_scores(g, b, d_qi, d_w, d_k, T, scores, T)
    sel = torch.full((n_q, sel_ld), -9, dtype=torch.int32, device=dev)
    cnt = torch.zeros(n_q, dtype=torch.int32, device=dev)
    out = torch.empty((n_q, 64, 512), device=dev)
    lse = torch.empty((n_q, 64), device=dev)
    d_q = torch.from_numpy(q.view(np.int16)).to(dev)
    d_c = torch.from_numpy(cache.view(np.int16)).to(dev)
    B.decode_step(g, b, d_qi, d_w, d_k, T, d_q, d_c, T, sel, sel_ld, cnt, out, lse, ws)
    torch.cuda.synchronize()
    qi = d_qi.cpu().numpy().view(np.uint16)
    keys = d_k.cpu().numpy().view(np.uint16)
    _check_prepared(qi[:2].reshape(-1, DI), q_in[:2].reshape(-1, DI), np.repeat(q_nvis[:2].astype(np.int64) - 1, HI),
                    f16, "step queries")
    _check_prepared(keys[1, ::97], k_in[T::97], k_pos[T::97], f16, "step keys (sampled)")
    ref_s = O.index_scores(q_seq, q_nvis, 1, qi, w_idx, keys, f16=True if f16 else False)
    got_s = scores.cpu().numpy()
    sel_g, cnt_g = sel.cpu().numpy(), cnt.cpu().numpy()
    kf = _decode16(keys, f16)
    qf = _decode16(qi, f16)
    top_k = g["top_k"]
    for j in range(n_q):
        rows = int(q_nvis[j])
        kk = kf[q_seq[j], :rows]
        bound = 2.0 ** -20 * (np.abs(kk) @ np.abs(qf[j]).T) @ w_idx[j].astype(np.float64)
        err = np.abs(got_s[j, :rows].astype(np.float64) - ref_s[j, :rows].astype(np.float64))
        assert (err <= bound).all(), f"query {j}: score error {err.max():.3e} over its bound"
        order = np.lexsort((np.arange(rows), -ref_s[j, :rows].astype(np.float64)))
        thr = float(ref_s[j, order[top_k - 1]])
        want = set(order[:top_k].tolist())
        have = set(sel_g[j, :cnt_g[j]].tolist())
        assert cnt_g[j] == top_k and len(have) == top_k
        for r in want ^ have:
            assert abs(float(ref_s[j, r]) - thr) <= 2 * bound[r], f"query {j}: row {r} differs away from a tie"
        log(f"query {j}: {len(want ^ have) // 2} near-tie swaps, max score error {err.max():.2e}")
    out_ref, lse_ref = O.mla_attend(q_seq, 512, 64, 1 / 16, q, cache, sel_g, cnt_g)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), out_ref, lse_ref, f"prepared step f16={f16}")
