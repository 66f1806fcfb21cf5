"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function takes an oracle library handle (``oracle.load``) and
raises AssertionError when the oracle disagrees with what the pages and the
mathematics fix: integer closed forms, an independent library routine
(numpy's integer matmul, ``lexsort``, float64 softmax), invariants and
hand-derived small cases.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on deliberately broken copies
of the oracle source and requires that every copy fails at least one pin.
"""
from __future__ import annotations

import math

import os

import numpy as np

from oracle import oracle as O
from deepseek_sparse_attention_amd.inputs import f32_to_bf16_bits, bf16_bits_to_f32

HI, DI, H = 32, 128, 64


def bf(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def fl(b):
    return bf16_bits_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------- brute force
def brute_scores(qi_int, w, K_int, rows):
    """s = relu(K qi^T) w in exact integer arithmetic (numpy int64 matmul)."""
    dots = K_int[:rows].astype(np.int64) @ qi_int.astype(np.int64).T      # [rows, HI]
    return np.maximum(dots, 0) @ w.astype(np.int64)


def brute_select(s, n_vis, kpool, top_k, ties_high=False, strict=False, tail=True,
                 dense_fallback=True, order="index"):
    """Reference selection by full lexsort.  Keyword switches give the rival
    readings that the pages' text leaves room for; the defaults are the
    reading the oracle implements."""
    rows, keep = n_vis // kpool, top_k // kpool
    if dense_fallback and rows <= keep:
        return list(range(n_vis))
    idx = np.arange(rows)
    sc = np.asarray(s[:rows], dtype=np.float64)
    if ties_high:
        order_ = np.lexsort((-idx, -sc))
    else:
        order_ = np.lexsort((idx, -sc))
    picked = order_[:min(keep, rows)]
    if strict:   # keep only rows strictly above the keep-th score
        thr = sc[order_[min(keep, rows) - 1]]
        picked = idx[sc > thr]
    if order == "index":
        picked = np.sort(picked)
    out = [int(p) * kpool + j for p in picked for j in range(kpool)]
    if tail:
        out += list(range(rows * kpool, n_vis))
    return out


def brute_attend(qh, C, sel, scale, d_latent):
    """Softmax attention of one head over selected rows, float64."""
    rows = C[np.asarray(sel)]
    z = scale * (rows @ qh)
    m = z.max()
    p = np.exp(z - m)
    o = (p @ rows[:, :d_latent]) / p.sum()
    return o, m + math.log(p.sum())


# ---------------------------------------------------------------- scores
def pin_scores_integer_closed_form(L):
    """Integer inputs: the score is exact, so it must equal the int64 brute
    force bit for bit, for tokens and for pools, with negative and zero head
    weights (which separate ReLU-then-weight from weight-then-ReLU)."""
    rng = np.random.default_rng(101)
    for kpool, key_rows, nvis in ((1, 300, [300, 257, 1]), (4, 75, [300, 259, 7])):
        qi = rng.integers(-8, 9, size=(3, HI, DI))
        K = rng.integers(-8, 9, size=(2, key_rows, DI))
        w = rng.integers(-2, 5, size=(3, HI))
        q_seq = np.array([0, 1, 1])
        s = O.index_scores(q_seq, nvis, kpool, bf(qi), w.astype(np.float32), bf(K), L=L)
        for j in range(3):
            rows = nvis[j] // kpool
            ref = brute_scores(qi[j], w[j], K[q_seq[j]], rows)
            assert np.array_equal(s[j, :rows], ref.astype(np.float32)), (kpool, j)
            assert np.isnan(s[j, rows:]).all(), "wrote past the visible rows"


def pin_scores_hand_case(L):
    """Two active heads, hand-derived: head 0 has q=2 at d=0 and weight 3,
    head 1 has q=-1 at d=1 and weight 5; key r has k[0]=r-2, k[1]=1-r.
    s(r) = 3*max(0, 2(r-2)) + 5*max(0, r-1) = 0, 0, 5, 16, 27 for r=0..4."""
    qi = np.zeros((1, HI, DI))
    qi[0, 0, 0], qi[0, 1, 1] = 2, -1
    w = np.zeros((1, HI), dtype=np.float32)
    w[0, 0], w[0, 1] = 3, 5
    K = np.zeros((1, 5, DI))
    K[0, :, 0] = np.arange(5) - 2
    K[0, :, 1] = 1 - np.arange(5)
    s = O.index_scores([0], [5], 1, bf(qi), w, bf(K), L=L)
    assert s[0].tolist() == [0.0, 0.0, 5.0, 16.0, 27.0], s


def pin_scores_real_valued(L):
    """Real-valued inputs: equal to a float64 numpy evaluation rounded once."""
    rng = np.random.default_rng(7)
    qi = fl(bf(rng.standard_normal((2, HI, DI))))
    K = fl(bf(rng.standard_normal((1, 64, DI))))
    w = rng.standard_normal((2, HI)).astype(np.float32)
    s = O.index_scores([0, 0], [64, 33], 1, bf(qi), w, bf(K), L=L)
    for j, rows in enumerate((64, 33)):
        ref = np.maximum(K[0, :rows] @ qi[j].T, 0) @ w[j].astype(np.float64)
        assert np.allclose(s[j, :rows], ref, rtol=1e-6, atol=1e-5)


# ---------------------------------------------------------------- top-k
def _check_topk_against_brute(L, s_rows, n_vis, kpool, top_k):
    n_q = len(n_vis)
    sel, cnt = O.topk(n_vis, kpool, top_k, s_rows, L=L)
    for j in range(n_q):
        ref = brute_select(s_rows[j], n_vis[j], kpool, top_k)
        got = sel[j, :cnt[j]].tolist()
        assert got == ref, (kpool, top_k, n_vis[j], got[:16], ref[:16])
        assert (sel[j, cnt[j]:] == -1).all()


def pin_topk_straddle_sweep(L):
    """Every visible count around the budget, token and pool level, with
    score vectors full of equal values (ties resolved by lower index)."""
    rng = np.random.default_rng(5)
    for kpool, tops in ((1, (1, 2, 3, 8, 16, 64)), (4, (4, 8, 16, 64))):
        for top_k in tops:
            keep = top_k // kpool
            lo = max(1, (keep - 3) * kpool)
            hi = (keep + 4) * kpool + kpool
            n_vis = list(range(lo, hi + 1))
            rows_max = max(n_vis) // kpool
            s = rng.integers(0, 4, size=(len(n_vis), max(rows_max, 1))).astype(np.float32)
            _check_topk_against_brute(L, s, n_vis, kpool, top_k)


def pin_topk_large_random(L):
    """Larger random cases, real and integer valued, against lexsort."""
    rng = np.random.default_rng(9)
    s_real = rng.standard_normal((3, 5000)).astype(np.float32)
    _check_topk_against_brute(L, s_real, [5000, 4097, 2049], 1, 2048)
    s_int = rng.integers(0, 50, size=(3, 5000)).astype(np.float32)
    _check_topk_against_brute(L, s_int, [5000, 4999, 3000], 1, 2048)
    s_pool = rng.integers(0, 20, size=(2, 1300)).astype(np.float32)
    _check_topk_against_brute(L, s_pool, [5203, 2052], 4, 2048)


def pin_topk_signed_zero(L):
    """-0.0 and +0.0 are the same score: the lower index wins the tie."""
    s = np.array([[-0.0, 0.0, -0.0, 1.0, 0.0]], dtype=np.float32)
    sel, cnt = O.topk([5], 1, 3, s, L=L)
    assert sel[0, :cnt[0]].tolist() == [0, 1, 3]


def pin_topk_written_rows(L):
    """Hand-written expected rows; each fixture also separates the oracle's
    reading from a rival one that the pages leave room for."""
    s = np.array([[5, 7, 7, 1, 7, 0, 3, 7]], dtype=np.float32)
    sel, cnt = O.topk([8], 1, 3, s, L=L)
    assert sel[0, :cnt[0]].tolist() == [1, 2, 4]
    assert brute_select(s[0], 8, 1, 3, ties_high=True) == [2, 4, 7]
    assert brute_select(s[0], 8, 1, 3, strict=True) == []        # all four 7s tie at the k-th
    assert brute_select(s[0], 8, 1, 3, order="score") == [1, 2, 4]
    s2 = np.array([[1, 9, 4, 9, 2, 8]], dtype=np.float32)
    sel, cnt = O.topk([6], 1, 3, s2, L=L)
    assert sel[0, :cnt[0]].tolist() == [1, 3, 5]
    assert brute_select(s2[0], 6, 1, 3, strict=True) == [1, 3]
    # pools of 4, keep one pool: equal pool scores go to pool 0; tail appended
    sp = np.array([[3, 3]], dtype=np.float32)
    sel, cnt = O.topk([11], 4, 4, sp, L=L)
    assert sel[0, :cnt[0]].tolist() == [0, 1, 2, 3, 8, 9, 10]
    assert brute_select(sp[0], 11, 4, 4, ties_high=True) == [4, 5, 6, 7, 8, 9, 10]
    assert brute_select(sp[0], 11, 4, 4, tail=False) == [0, 1, 2, 3]
    # exactly at the budget: dense, every visible token including the tail
    sel, cnt = O.topk([7], 4, 4, np.array([[1.0]], dtype=np.float32), L=L)
    assert sel[0, :cnt[0]].tolist() == list(range(7))
    sel, cnt = O.topk([8], 4, 4, np.array([[1.0, 2.0]], dtype=np.float32), L=L)
    assert sel[0, :cnt[0]].tolist() == [4, 5, 6, 7]
    # dense below k at token level, whatever the scores
    sel, cnt = O.topk([3], 1, 4, np.array([[9.0, -1.0, 2.0]], dtype=np.float32), L=L)
    assert sel[0, :cnt[0]].tolist() == [0, 1, 2]
    assert brute_select([9.0, -1.0, 2.0], 3, 1, 4, dense_fallback=False) == [0, 1, 2]


def _golden(name):
    """key -> list of int values of a tests/golden fixture (# lines are
    comments; a line is a key followed by values, or key value pairs)."""
    out = {}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if not line:
                continue
            if len(line) == 2:
                out[line[0]] = int(line[1])
            else:
                for k, v in zip(line[0::2], line[1::2]):
                    out[k] = int(v)
    return out


def pin_topk_kpool_branch_from_the_pages(L):
    """The pages' worked case (tests/golden/kpool_branch_2100.txt): over a
    2,100-token prompt the k-pool selection is sparse exactly at positions
    2051..2099, and at 2,052 cached tokens keeps 512 of 513 pools = 2,048
    pooled positions (no tail).  Scores are random pool scores."""
    g = _golden("kpool_branch_2100.txt")
    kp, k, T = g["kpool"], g["top_k"], g["prompt_tokens"]
    rng = np.random.default_rng(2100)
    n_vis = np.arange(1, T + 1, dtype=np.int32)              # position p sees p + 1 tokens
    s = rng.standard_normal((T, T // kp)).astype(np.float32)
    sel, cnt = O.topk(n_vis, kp, k, s, L=L)
    sparse = [p for p in range(T) if cnt[p] < n_vis[p]]
    assert sparse == list(range(g["first_sparse_position"], g["last_sparse_position"] + 1))
    p = g["at_cached"] - 1
    rows = sel[p, :cnt[p]]
    assert g["at_cached"] // kp == g["complete_pools"]
    assert cnt[p] == g["pooled_positions"] and len(set((rows // kp).tolist())) == g["kept_pools"]
    # every kept pool whole, and exactly the best pools by (score desc, pool asc)
    pools = np.unique(rows // kp)
    assert np.array_equal(np.sort(rows), np.sort((pools[:, None] * kp + np.arange(kp)).ravel()))
    order = np.lexsort((np.arange(g["complete_pools"]), -s[p, :g["complete_pools"]]))
    assert np.array_equal(pools, np.sort(order[:g["kept_pools"]]))


def pin_topk_invariants(L):
    """|S| = min(k, n); every selected score >= every unselected one; among
    scores equal to the smallest selected one, the selected have the lowest
    indices."""
    rng = np.random.default_rng(11)
    n, k = 6000, 2048
    s = rng.integers(0, 300, size=(1, n)).astype(np.float32)
    sel, cnt = O.topk([n], 1, k, s, L=L)
    S = sel[0, :cnt[0]]
    assert cnt[0] == k and len(set(S.tolist())) == k
    mask = np.zeros(n, bool)
    mask[S] = True
    thr = s[0, S].min()
    assert s[0, mask].min() >= s[0, ~mask].max()
    eq = np.nonzero(s[0] == thr)[0]
    taken = eq[mask[eq]]
    assert (taken == eq[:len(taken)]).all()


# ---------------------------------------------------------------- attention
def pin_attend_dense_matches_softmax(L):
    """k >= n_vis: attention over the selection is dense masked softmax
    attention, computed independently in float64 with numpy."""
    rng = np.random.default_rng(3)
    T, D, dl = 100, 576, 512
    C = bf(rng.standard_normal((2, T, D)))
    q = bf(rng.standard_normal((2, H, D)))
    sel = np.full((2, 2048), -1, np.int32)
    sel[0, :100] = np.arange(100)
    picks = np.sort(rng.choice(T, 37, replace=False))
    sel[1, :37] = picks
    cnt = np.array([100, 37], np.int32)
    out, lse = O.mla_attend([0, 1], dl, 64, 1 / 16, q, C, sel, cnt, L=L)
    Cf, qf = fl(C), fl(q)
    for j, (s_, c_) in enumerate(((0, sel[0, :100]), (1, picks))):
        for h in range(H):
            o, l_ = brute_attend(qf[j, h], Cf[s_], c_, 1 / 16, dl)
            assert np.allclose(out[j, h], o, rtol=1e-5, atol=1e-6), (j, h)
            assert abs(lse[j, h] - l_) < 1e-5 * max(1.0, abs(l_))


def pin_attend_constant_v(L):
    """Rows whose latent part is one vector v: the output is v (the softmax
    weights sum to one), whatever the scores."""
    rng = np.random.default_rng(4)
    T, D, dl = 40, 576, 512
    v = rng.standard_normal(dl)
    C = rng.standard_normal((1, T, D))
    C[0, :, :dl] = v
    q = bf(rng.standard_normal((1, H, D)) * 3)
    sel = np.full((1, 64), -1, np.int32)
    sel[0, :T] = np.arange(T)
    out, _ = O.mla_attend([0], dl, 64, 1 / 16, q, bf(C), sel, [T], L=L)
    assert np.allclose(out[0], fl(bf(v))[None, :], rtol=1e-6, atol=1e-7)


def pin_attend_two_token_scale(L):
    """q = 16 e_0, rows e_0 and e_1: z = (1, 0) with scale 1/16, so
    o = (sigmoid(1), 1 - sigmoid(1), 0, ...) and lse = log(1 + e).  Scale
    1/sqrt(512) or 1/sqrt(576) would give 0.67 instead of 0.731."""
    D, dl = 576, 512
    C = np.zeros((1, 2, D))
    C[0, 0, 0] = 1
    C[0, 1, 1] = 1
    q = np.zeros((1, H, D))
    q[0, :, 0] = 16
    sel = np.array([[0, 1]], np.int32)
    out, lse = O.mla_attend([0], dl, 64, 1 / 16, bf(q), bf(C), sel, [2], L=L)
    sig = 1 / (1 + math.exp(-1))
    assert abs(out[0, 0, 0] - 0.7310585786) < 1e-7 and abs(out[0, 0, 0] - sig) < 1e-7
    assert abs(out[0, 0, 1] - (1 - sig)) < 1e-7
    assert np.all(out[0, :, 2:] == 0)
    assert abs(lse[0, 0] - math.log(1 + math.e)) < 1e-6


def pin_attend_rope_part_scores(L):
    """The 64-wide RoPE tail takes part in the score but not in V: with equal
    latent scores and q = 16 on the first rope column, rows with rope 1 and 0
    weigh sigmoid(1) and 1 - sigmoid(1); the output carries only latents."""
    D, dl = 576, 512
    C = np.zeros((1, 2, D))
    C[0, 0, 0], C[0, 1, 1] = 1, 1
    C[0, 0, dl] = 1                 # rope column 0 of row 0
    C[0, :, dl + 1] = 5             # equal in both rows
    q = np.zeros((1, H, D))
    q[0, :, dl] = 16
    q[0, :, dl + 1] = 2
    sel = np.array([[0, 1]], np.int32)
    out, _ = O.mla_attend([0], dl, 64, 1 / 16, bf(q), bf(C), sel, [2], L=L)
    sig = 1 / (1 + math.exp(-1))
    assert abs(out[0, 3, 0] - sig) < 1e-7 and abs(out[0, 3, 1] - (1 - sig)) < 1e-7


def pin_attend_nope(L):
    """NoPE rows (d_rope = 0): K = V = the 512-wide latent; float64 numpy."""
    rng = np.random.default_rng(6)
    T, dl = 50, 512
    C = bf(rng.standard_normal((1, T, dl)))
    q = bf(rng.standard_normal((1, H, dl)))
    picks = np.array([1, 4, 9, 10, 11, 12, 30, 49], np.int32)
    sel = np.full((1, 2051), -1, np.int32)
    sel[0, :8] = picks
    out, lse = O.mla_attend([0], dl, 0, 1 / 16, q, C, sel, [8], L=L)
    for h in range(H):
        o, l_ = brute_attend(fl(q)[0, h], fl(C)[0], picks, 1 / 16, dl)
        assert np.allclose(out[0, h], o, rtol=1e-5, atol=1e-6)
        assert abs(lse[0, h] - l_) < 1e-5 * max(1.0, abs(l_))


# ---------------------------------------------------------------- fused step
def pin_decode_is_composition(L):
    """The fused step equals scores -> top-k -> attention, and a prefill
    chunk equals one decode per position with n_vis = position + 1."""
    rng = np.random.default_rng(8)
    geom = dict(n_heads=H, d_latent=512, d_rope=64, n_idx_heads=HI, d_idx=DI,
                top_k=16, kpool=1, softmax_scale=1 / 16)
    T = 40
    C = bf(rng.standard_normal((1, T, 576)))
    K = bf(rng.integers(-8, 9, size=(1, T, DI)))
    nq = 6
    nvis = np.array([10, 16, 17, 25, 39, 40], np.int32)
    qseq = np.zeros(nq, np.int32)
    qi = bf(rng.integers(-8, 9, size=(nq, HI, DI)))
    w = rng.integers(1, 5, size=(nq, HI)).astype(np.float32)
    q = bf(rng.standard_normal((nq, H, 576)))
    sel, cnt, out, lse = O.decode_step(geom, qseq, nvis, qi, w, K, q, C, L=L)
    s = O.index_scores(qseq, nvis, 1, qi, w, K, L=L)
    sel2, cnt2 = O.topk(nvis, 1, 16, s, L=L)
    out2, lse2 = O.mla_attend(qseq, 512, 64, 1 / 16, q, C, sel2, cnt2, L=L)
    assert np.array_equal(sel, sel2) and np.array_equal(cnt, cnt2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    for j in range(nq):
        r = brute_select(brute_scores(fl(qi)[j].astype(np.int64), w[j].astype(np.int64),
                                      fl(K)[0].astype(np.int64), nvis[j]), nvis[j], 1, 16)
        assert sel[j, :cnt[j]].tolist() == r
        s1, c1, o1, l1 = O.decode_step(geom, [0], nvis[j:j + 1], qi[j:j + 1], w[j:j + 1],
                                       K, q[j:j + 1], C, L=L)
        assert np.array_equal(o1[0], out[j]) and np.array_equal(s1[0], sel[j])


# ---------------------------------------------------------------- pool keys
def _pool_one(L, keys4, gates4, pos_emb):
    """Key of one pool from four cells, through the oracle's append."""
    kg = np.concatenate([bf(keys4), bf(gates4)], axis=-1)[None]        # [1, 4, 2 DI]
    roll = np.zeros((1, 4, 2 * DI), np.uint16)
    pk = np.zeros((1, 1, DI), np.uint16)
    O.pool_append([0], [4], kg, roll, pk, np.asarray(pos_emb, np.float32), L=L)
    return pk[0, 0]


def pin_pool_equal_logits_give_mean(L):
    """Logits equal over the four slots weight them equally, so the pool key
    is the mean of the four keys (exact for integer keys: a multiple of 1/4)."""
    rng = np.random.default_rng(31)
    keys = rng.integers(-8, 9, size=(4, DI)).astype(np.float32)
    gates = np.tile(rng.standard_normal(DI).astype(np.float32), (4, 1))
    assert np.array_equal(fl(_pool_one(L, keys, gates, np.zeros((4, DI)))), keys.mean(0))
    pos = np.tile(rng.standard_normal(DI).astype(np.float32), (4, 1))
    assert np.array_equal(fl(_pool_one(L, keys, gates, pos)), keys.mean(0))


def pin_pool_dominant_slot(L):
    """A slot whose logit exceeds the others' by 800 takes all the weight
    (exp(-800) underflows to 0), per key dimension: the pool key is that
    slot's key, whether the margin comes from the gate or from the slot's
    position embedding."""
    rng = np.random.default_rng(32)
    keys = rng.integers(-8, 9, size=(4, DI)).astype(np.float32)
    dom = (np.arange(DI) * 7 + 3) % 4
    want = keys[dom, np.arange(DI)]
    gates = np.zeros((4, DI), np.float32)
    gates[dom, np.arange(DI)] = 800.0
    assert np.array_equal(fl(_pool_one(L, keys, gates, np.zeros((4, DI)))), want)
    pos = np.zeros((4, DI), np.float32)
    pos[dom, np.arange(DI)] = 800.0
    assert np.array_equal(fl(_pool_one(L, keys, np.zeros((4, DI)), pos)), want)


def pin_pool_constant_keys(L):
    """Four equal keys give that key under any weights."""
    rng = np.random.default_rng(33)
    c = fl(bf(rng.standard_normal(DI)))
    out = _pool_one(L, np.tile(c, (4, 1)), rng.standard_normal((4, DI)) * 3, rng.standard_normal((4, DI)))
    assert np.array_equal(fl(out), c)


def pin_pool_convex_and_shift_invariant(L):
    """The pool key lies between the smallest and largest of the four keys in
    every dimension, and adding one constant to every slot's logit of a
    dimension changes nothing (softmax shift invariance)."""
    rng = np.random.default_rng(34)
    for _ in range(20):
        keys = fl(bf(rng.standard_normal((4, DI)) * 4))
        gates = rng.standard_normal((4, DI)) * 2
        pos = np.round(rng.standard_normal((4, DI)) * 256) / 256       # exact in float32
        out = fl(_pool_one(L, keys, gates, pos))
        assert (out >= keys.min(0)).all() and (out <= keys.max(0)).all()
        shift = np.tile(np.round(rng.standard_normal(DI)) * 2, (4, 1))  # even integers: sums stay exact
        assert np.array_equal(fl(_pool_one(L, keys, gates, pos + shift)), out)


def pin_pool_rounding(L):
    """The stored key is the nearest bf16, ties to even: with equal logits,
    keys (1+2^-7, 1+2^-7, 1+2^-7, 1) average 1 + 3*2^-9 -> 1+2^-7, and
    (1+2^-7, 1+2^-7, 1, 1) average 1 + 2^-8, halfway -> 1 (even)."""
    a, b = 1.0 + 2.0 ** -7, 1.0
    g = np.zeros((4, DI))
    z = np.zeros((4, DI))
    up = _pool_one(L, np.array([[a], [a], [a], [b]]) * np.ones((4, DI)), g, z)
    tie = _pool_one(L, np.array([[a], [a], [b], [b]]) * np.ones((4, DI)), g, z)
    neg = _pool_one(L, -np.array([[a], [a], [a], [b]]) * np.ones((4, DI)), g, z)
    assert (fl(up) == a).all() and (fl(tie) == b).all() and (fl(neg) == -a).all()


def pin_pool_append_semantics(L):
    """Appending tokens one by one, in chunks or all at once gives the same
    pool keys and rolling buffer; pool p depends on cells 4p..4p+3 only; the
    rolling buffer holds the cells of the pool being filled at slot t mod 4;
    pools not yet complete are not written."""
    rng = np.random.default_rng(35)
    n = np.array([23, 14, 3], np.int32)
    cells = np.concatenate([bf(rng.standard_normal((3, 23, DI)) * 3),
                            bf(rng.standard_normal((3, 23, DI)))], axis=-1)
    pos = rng.standard_normal((4, DI)).astype(np.float32)
    SENT = 0x7F7F

    def run(chunks):
        roll = np.zeros((3, 4, 2 * DI), np.uint16)
        pk = np.full((3, 6, DI), SENT, np.uint16)
        done = np.zeros(3, np.int32)
        for c in chunks:
            take = np.minimum(c, n - done)
            kg = np.zeros((3, max(1, int(take.max())), 2 * DI), np.uint16)
            for s_ in range(3):
                kg[s_, :take[s_]] = cells[s_, done[s_]:done[s_] + take[s_]]
            O.pool_append(done, take, kg, roll, pk, pos, L=L)
            done += take
        assert np.array_equal(done, n)
        return roll, pk

    r1, p1 = run([np.ones(3, np.int32)] * 23)
    r2, p2 = run([np.array([5, 2, 1]), np.array([7, 9, 1]), np.array([11, 3, 1])])
    r3, p3 = run([n.copy()])
    assert np.array_equal(r1, r2) and np.array_equal(r1, r3)
    assert np.array_equal(p1, p2) and np.array_equal(p1, p3)
    for s_ in range(3):
        for p_ in range(6):
            if p_ < n[s_] // 4:
                c4 = cells[s_, 4 * p_:4 * p_ + 4]
                assert np.array_equal(p1[s_, p_], _pool_one(L, fl(c4[:, :DI]), fl(c4[:, DI:]), pos))
            else:
                assert (p1[s_, p_] == SENT).all()
        for t in range(4 * (n[s_] // 4), n[s_]):
            assert np.array_equal(r1[s_, t % 4], cells[s_, t])


# ---------------------------------------------------------------- absorption
DN, DL, DV = 256, 512, 256


def _sparse_unit(rng, shape, density):
    """Entries in {-1, 0, 1}, mostly 0: sums stay small integers, exact in bf16."""
    v = rng.integers(-1, 2, size=shape) * (rng.random(shape) < density)
    return v.astype(np.float32)


def pin_absorb_is_the_key_identity(L):
    """By linearity q . (W L) = (W^T q) . L: the absorbed query dotted with a
    latent row equals the query dotted with the decompressed key, computed
    here by numpy integer matmuls (small integers, so every value is exact)."""
    rng = np.random.default_rng(41)
    n_q, Hh, T = 3, 4, 9
    qn = _sparse_unit(rng, (n_q, Hh, DN), 0.05)
    W = _sparse_unit(rng, (Hh, DN, DL), 0.01)
    Lat = rng.integers(-3, 4, size=(T, DL)).astype(np.int64)
    qa = fl(O.absorb_query(bf(qn), None, bf(W), L=L))                    # [n_q, H, DL]
    assert np.array_equal(qa, np.einsum("mhk,hkn->mhn", qn.astype(np.int64), W.astype(np.int64)))
    keys = np.einsum("hkn,tn->htk", W.astype(np.int64), Lat)              # decompressed keys
    for m in range(n_q):
        for h in range(Hh):
            assert np.array_equal(qa[m, h].astype(np.int64) @ Lat.T, keys[h] @ qn[m, h].astype(np.int64))


def pin_absorb_selection_and_rope(L):
    """W = [I | 0] puts q_nope in the first 256 latent dimensions; the RoPE
    part is appended unchanged after the 512 latent dimensions."""
    rng = np.random.default_rng(42)
    qn = bf(rng.standard_normal((2, 3, DN)))
    qr = bf(rng.standard_normal((2, 3, 64)))
    W = np.zeros((3, DN, DL), np.float32)
    W[:, np.arange(DN), np.arange(DN)] = 1.0
    qa = O.absorb_query(qn, qr, bf(W), L=L)
    assert np.array_equal(qa[:, :, :DN], qn) and (fl(qa[:, :, DN:DL]) == 0).all()
    assert np.array_equal(qa[:, :, DL:], qr)


def pin_absorb_rounding(L):
    """The absorbed query is the nearest bf16 of the exact sum, ties to even:
    1 + 2^-7 + 2^-9 -> 1 + 2^-7; 1 + 2^-7 + 3*2^-9 -> 1 + 2^-6; and the tie
    1 + 2^-7 + 2^-8 -> 1 + 2^-6 (even)."""
    def one(extra):
        qn = np.zeros((1, 1, DN), np.float32)
        qn[0, 0, :2] = [1.0, 1.0]
        W = np.zeros((1, DN, DL), np.float32)
        W[0, 0, 0] = 1.0 + 2.0 ** -7
        W[0, 1, 0] = extra
        return float(fl(O.absorb_query(bf(qn), None, bf(W), L=L))[0, 0, 0])
    assert one(2.0 ** -9) == 1.0 + 2.0 ** -7
    assert one(3 * 2.0 ** -9) == 1.0 + 2.0 ** -6
    assert one(2.0 ** -8) == 1.0 + 2.0 ** -6


def pin_project_selection_and_linearity(L):
    """W_UV = [I | 0] returns the first 256 latent columns; the projection is
    linear (exact for integer-valued inputs) and matches float64 matmul."""
    rng = np.random.default_rng(43)
    o = rng.standard_normal((2, 3, DL)).astype(np.float32)
    W = np.zeros((3, DV, DL), np.float32)
    W[:, np.arange(DV), np.arange(DV)] = 1.0
    assert np.array_equal(O.project_output(o, bf(W), L=L), o[:, :, :DV])
    oi = rng.integers(-8, 9, size=(2, 3, DL)).astype(np.float32)
    oj = rng.integers(-8, 9, size=(2, 3, DL)).astype(np.float32)
    Wi = bf(rng.integers(-4, 5, size=(3, DV, DL)))
    assert np.array_equal(O.project_output(oi + oj, Wi, L=L),
                          O.project_output(oi, Wi, L=L) + O.project_output(oj, Wi, L=L))
    Wr = bf(rng.standard_normal((3, DV, DL)))
    ref = np.einsum("mhj,hij->mhi", o.astype(np.float64), fl(Wr))
    assert np.allclose(O.project_output(o, Wr, L=L), ref, rtol=1e-6, atol=1e-5)


def pin_absorbed_attention_is_explicit_mla(L):
    """Absorbed decode equals explicit MLA: per head, keys k_t = W_UK L_t and
    values v_t = W_UV L_t decompressed from the latent, scores
    (q_nope . k_t + q_rope . rope_t) / 16, softmax, output sum_t p_t v_t
    (float64 numpy; the absorbed path rounds q_abs to bf16, hence the
    tolerance)."""
    rng = np.random.default_rng(44)
    Hh, T, n_q = 64, 12, 2
    qn = bf(rng.standard_normal((n_q, Hh, DN)) * 0.5)
    qr = bf(rng.standard_normal((n_q, Hh, 64)))
    Wk = bf(rng.standard_normal((Hh, DN, DL)) * 0.05)
    Wv = bf(rng.standard_normal((Hh, DV, DL)) * 0.05)
    C = bf(rng.standard_normal((1, T, DL + 64)))
    qa = O.absorb_query(qn, qr, Wk, L=L)
    sel = np.tile(np.arange(T, dtype=np.int32), (n_q, 1))
    o, _ = O.mla_attend(np.zeros(n_q, np.int32), DL, 64, 1 / 16, qa, C, sel, np.full(n_q, T, np.int32), L=L)
    ctx = O.project_output(o, Wv, L=L)
    Lt, rope = fl(C[0, :, :DL]), fl(C[0, :, DL:])
    for m in range(n_q):
        for h in range(Hh):
            k = Lt @ fl(Wk[h]).T                                 # [T, DN]
            v = Lt @ fl(Wv[h]).T                                 # [T, DV]
            z = (k @ fl(qn[m, h]) + rope @ fl(qr[m, h])) / 16
            p = np.exp(z - z.max())
            p /= p.sum()
            want = p @ v
            assert np.allclose(ctx[m, h], want, rtol=2e-3, atol=2e-3 * np.abs(want).max())


# ---------------------------------------------------------------- indexer input preparation
BASE = 8.0e6          # RoPE base of the pages' model table


def _sylvester():
    """Orthonormal Walsh-Hadamard matrix from scipy (Sylvester order)."""
    import scipy.linalg
    return scipy.linalg.hadamard(DI).astype(np.float64) / math.sqrt(DI)


def pin_prep_rotation_is_library_hadamard(L):
    """Without rope (or at position 0, where rope turns by zero) the rotation
    is scipy's Sylvester Hadamard matrix scaled by 1/sqrt(128)."""
    Hm = _sylvester()
    rng = np.random.default_rng(31)
    for _ in range(3):
        x = rng.standard_normal(DI)
        assert np.allclose(O.index_rotate(x, 777, 0, L=L), Hm @ x, rtol=0, atol=1e-12)
        assert np.allclose(O.index_rotate(x, 0, 64, L=L), Hm @ x, rtol=0, atol=1e-12)
    e0 = np.zeros(DI)
    e0[0] = 1.0
    assert np.allclose(O.index_rotate(e0, 5, 0, L=L), np.full(DI, 1 / math.sqrt(DI)), atol=1e-15)


def pin_prep_rotation_orthonormal_involution(L):
    """The Hadamard rotation is orthonormal and its own inverse; with rope at
    any position the map still preserves the norm (rope is a rotation)."""
    rng = np.random.default_rng(32)
    for pos in (1, 4097, 1048575):
        x = rng.standard_normal(DI) * 3
        y = O.index_rotate(x, 0, 0, L=L)
        assert np.allclose(O.index_rotate(y, 0, 0, L=L), x, atol=1e-12)
        z = O.index_rotate(x, pos, 64, L=L)
        assert abs(np.linalg.norm(z) - np.linalg.norm(x)) < 1e-12 * np.linalg.norm(x)


def pin_prep_rope_pairs_and_frequencies(L):
    """Undoing the Hadamard rotation (scipy's matrix, its own inverse) leaves
    the rope alone: the first 64 dimensions are untouched at any position;
    the unit vector on dimension 64+2j stays in the pair (64+2j, 65+2j) and
    turns counter-clockwise by p * base^(-2j/64).  Pair 0 turns by exactly p
    radians; the angles at p = 1 form a geometric series of ratio
    base^(-1/32)."""
    Hm = _sylvester()
    rng = np.random.default_rng(33)
    x = rng.standard_normal(DI)
    for pos in (1, 3, 131071):
        r = Hm @ O.index_rotate(x, pos, 64, L=L)
        assert np.allclose(r[:64], x[:64], atol=1e-12)
    ang = []
    for j in range(32):
        e = np.zeros(DI)
        e[64 + 2 * j] = 1.0
        r = Hm @ O.index_rotate(e, 1, 64, L=L)
        rest = np.delete(r, [64 + 2 * j, 65 + 2 * j])
        assert np.abs(rest).max() < 1e-12, j
        ang.append(math.atan2(r[65 + 2 * j], r[64 + 2 * j]))
    ang = np.array(ang)
    assert abs(ang[0] - 1.0) < 1e-12
    assert np.allclose(ang[1:] / ang[:-1], BASE ** (-1.0 / 32), rtol=1e-9)
    assert abs(ang[31] - BASE ** (-62.0 / 64)) < 1e-15
    e = np.zeros(DI)
    e[64] = 1.0
    r = Hm @ O.index_rotate(e, 2, 64, L=L)
    assert abs(r[64] - math.cos(2.0)) < 1e-12 and abs(r[65] - math.sin(2.0)) < 1e-12


def pin_prep_relative_position(L):
    """Rope makes the score depend on the distance only, and the rotation
    applied to both sides cancels: q(p).k(s) == q(p+d).k(s+d), and equals
    q.k when p == s."""
    rng = np.random.default_rng(34)
    q, k = rng.standard_normal(DI), rng.standard_normal(DI)
    for p, s_, d in ((10, 3, 1000), (0, 70000, 12345)):
        a = O.index_rotate(q, p, 64, L=L) @ O.index_rotate(k, s_, 64, L=L)
        b = O.index_rotate(q, p + d, 64, L=L) @ O.index_rotate(k, s_ + d, 64, L=L)
        assert abs(a - b) < 1e-9
    same = O.index_rotate(q, 4242, 64, L=L) @ O.index_rotate(k, 4242, 64, L=L)
    assert abs(same - q @ k) < 1e-10


def pin_prep_rounding(L):
    """f16 rounding equals numpy's float64 -> float16 conversion (nearest,
    ties to even, subnormals, overflow to infinity); bf16 ties go to even."""
    rng = np.random.default_rng(35)
    v = np.concatenate([
        rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -70000.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
         2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -(1 + 2.0 ** -11)]])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(O.round16(v, True, L=L), ref)
    b = O.round16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20]),
                  False, L=L)
    assert fl(b).tolist() == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]


def pin_prep_f16_scores(L):
    """Scores over f16 inputs equal a float64 evaluation of numpy's decoding
    of the same f16 bits (normal, subnormal and integer values)."""
    rng = np.random.default_rng(36)
    qi = (rng.standard_normal((2, HI, DI)) * 4).astype(np.float16)
    K = (rng.standard_normal((1, 80, DI)) * 2.0 ** rng.integers(-20, 4, (1, 80, 1))).astype(np.float16)
    w = rng.standard_normal((2, HI)).astype(np.float32)
    s = O.index_scores([0, 0], [80, 41], 1, qi.view(np.uint16), w, K.view(np.uint16), L=L, f16=True)
    for j, rows in enumerate((80, 41)):
        ref = np.maximum(K[0, :rows].astype(np.float64) @ qi[j].astype(np.float64).T, 0) @ w[j].astype(np.float64)
        assert np.allclose(s[j, :rows], ref, rtol=1e-6, atol=1e-30)
    # integer f16 inputs: exact, equal to the int64 brute force
    qz = rng.integers(-8, 9, size=(1, HI, DI))
    Kz = rng.integers(-8, 9, size=(1, 50, DI))
    wz = rng.integers(-2, 5, size=(1, HI))
    s = O.index_scores([0], [50], 1, qz.astype(np.float16).view(np.uint16), wz.astype(np.float32),
                       Kz.astype(np.float16).view(np.uint16), L=L, f16=True)
    assert np.array_equal(s[0], brute_scores(qz[0], wz[0], Kz[0], 50).astype(np.float32))


def pin_prep_positions_and_rows(L):
    """A query at n_vis = p + 1 sits at position p and a key appended at p
    sits at p: with both equal to one vector x whose energy is on rope pair
    0, q.k returns |x|^2 up to the 16-bit rounding (a position off by one
    turns pair 0 by a radian).  A query with n_vis = 1 is the plain
    rotation.  Keys land at row (seq, pos); a key whose sequence or position
    is out of range writes nothing; every other row is untouched."""
    Hm = _sylvester()
    rng = np.random.default_rng(37)
    n_seq, stride = 3, 40
    for f16 in (False, True):
        x = rng.standard_normal(DI) * 0.05
        x[64], x[65] = 6.0, 8.0
        q_in = np.stack([np.tile(x, (HI, 1)), rng.standard_normal((HI, DI))]).astype(np.float32)
        q_nvis = np.array([30, 1])
        k_pos = np.array([29, 0, 39, 40, -1, 5])
        k_seq = np.array([1, 0, 2, 0, 1, -1])
        k_in = np.stack([x] + [rng.standard_normal(DI) for _ in range(5)]).astype(np.float32)
        cache = np.full((n_seq, stride, DI), 0x1234, np.uint16)
        qo, cache = O.index_prepare(q_nvis, q_in, k_seq, k_pos, k_in, cache, 64, f16, L=L)
        dec = (lambda b: b.view(np.float16).astype(np.float64)) if f16 else fl
        dot = dec(qo[0, 5]) @ dec(cache[1, 29])
        assert abs(dot - x.astype(np.float32).astype(np.float64) @ x.astype(np.float32)) < 0.05 * 100 * 2 ** -6, dot
        plain = Hm @ q_in[1, 3].astype(np.float64)
        assert np.allclose(dec(qo[1, 3]), plain, rtol=2 ** -7, atol=1e-30)
        written = {(1, 29), (0, 0), (2, 39)}
        for s_ in range(n_seq):
            for r in range(stride):
                if (s_, r) not in written:
                    assert (cache[s_, r] == 0x1234).all(), (f16, s_, r)
        k0 = dec(cache[0, 0])
        assert np.allclose(k0, Hm @ k_in[1].astype(np.float64), rtol=2 ** -7, atol=1e-30)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
