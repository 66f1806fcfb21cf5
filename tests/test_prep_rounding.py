"""How the indexer's 16-bit rounding moves scores and selections, on the
CPU oracle alone (no GPU): the exact scores of rope'd projections against
those of the same vectors rounded to bf16 or f16, with and without the
Walsh-Hadamard rotation before the rounding.  With a few large channels the
rotation spreads their rounding error over all 128 dimensions and the score
error drops several times (TensorSharp2 GLM-5.x docs, section "The
sparse-attention path", report that skipping the rotation changed top-k
picks); f16 keeps three more fraction bits than bf16."""
from __future__ import annotations

import numpy as np
import scipy.linalg

from oracle import oracle as O
from deepseek_sparse_attention_amd import inputs as I

DI, HI, T, NQ, K = 128, 32, 8192, 3, 1024


def _decode(bits, f16):
    if f16:
        return bits.view(np.float16).astype(np.float64)
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def _scores(qv, kv, w):
    return np.stack([np.maximum(kv @ qv[j].T, 0) @ w[j] for j in range(qv.shape[0])])


def test_rotation_spreads_rounding_error():
    q_in, k_in = I.indexer_projections(5, NQ, T)
    w = np.random.default_rng(6).random((NQ, HI)) + 0.5
    kr = np.stack([O.index_rotate(k_in[i].astype(np.float64), i, 64) for i in range(T)])
    qr = np.stack([[O.index_rotate(q_in[j, h].astype(np.float64), T - 1, 64) for h in range(HI)]
                   for j in range(NQ)])
    Hm = scipy.linalg.hadamard(DI) / np.sqrt(DI)        # undoes the rotation (symmetric, orthonormal)
    exact = _scores(qr, kr, w)
    scale = np.abs(exact).max(axis=1, keepdims=True)
    top = [set(np.lexsort((np.arange(T), -exact[j]))[:K].tolist()) for j in range(NQ)]
    err = {}
    for f16 in (False, True):
        for rotated in (True, False):
            kv, qv = (kr, qr) if rotated else (kr @ Hm, qr @ Hm)
            s = _scores(_decode(O.round16(qv, f16), f16), _decode(O.round16(kv, f16), f16), w)
            e = float((np.abs(s - exact) / scale).max())
            moved = [len(top[j] - set(np.lexsort((np.arange(T), -s[j]))[:K].tolist())) for j in range(NQ)]
            err[(f16, rotated)] = e
            print(f"{'f16 ' if f16 else 'bf16'} {'rotated  ' if rotated else 'unrotated'}: "
                  f"max score error {e:.2e} of the row's largest, top-{K} picks moved {moved}")
    for f16 in (False, True):
        assert err[(f16, True)] * 2 < err[(f16, False)], "rotation did not spread the rounding error"
    assert err[(True, True)] * 4 < err[(False, True)], "f16 should round about 8x finer than bf16"
