"""Seeded synthetic inputs for the DSA decode hot path.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no scores, no ranking, no softmax), so both the HIP
path and the CPU oracle may be fed from it without sharing any computation.

The workloads follow the problem statement of the DeepSeek Sparse Attention
pages (GLM-5.x): a latent cache of 576-wide rows (512 latent columns, which
are also V, plus a 64-wide RoPE tail), 128-wide indexer keys, 64 absorbed
query heads of width 576, 32 indexer heads of width 128 with per-head weights,
and top-k 2048.  The k-pool NoPE variant has 512-wide rows and one indexer key
per pool of 4 tokens.

Recipe (stated once here, repeated in the design notes):
  * every tensor chunk draws from
    ``Generator(PCG64(SeedSequence([20261202, cfg_id, seq, tensor, chunk])))``
    with tensor ids 0 latent, 1 indexer keys, 2 query, 3 indexer query,
    4 head weights, 5 per-sequence offset; chunks are 16384 rows;
  * real-valued tensors are ``standard_normal(float32)`` rounded to bf16
    with round-to-nearest-even;
  * integer-valued tensors are ``integers(lo, hi + 1)``, which bf16 holds
    exactly;
  * head weights are ``integers(1, 5)`` stored as float32.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED = 20261202
T_LATENT, T_IDXK, T_Q, T_QI, T_W, T_OFF = range(6)
CHUNK_ROWS = 16384

BF16_NAN = np.uint16(0x7FC0)

# Geometry of token-level DSA (GLM-5.2/5.3) and of the pooled NoPE variant
# (GLM-5.3-Flash).  Keys are the fields of the C struct ``dsa_geometry``.
GEOM_TOKEN = dict(n_heads=64, d_latent=512, d_rope=64, n_idx_heads=32,
                  d_idx=128, top_k=2048, kpool=1, softmax_scale=1.0 / 16.0)
GEOM_KPOOL = dict(GEOM_TOKEN, d_rope=0, kpool=4)


def _rng(cfg_id: int, seq: int, tensor: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([SEED, cfg_id, seq, tensor, chunk])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _int_table() -> np.ndarray:
    # bf16 bit patterns of the integers -128..127 (all exact in bf16)
    return f32_to_bf16_bits(np.arange(-128, 128, dtype=np.float32))


_INT_BF16 = _int_table()


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclasses.dataclass
class Workload:
    """One batch of synthetic inputs in host memory (numpy)."""
    name: str
    cfg_id: int
    geom: dict
    n_seq: int
    T: int                # latent rows allocated per sequence
    key_rows: int         # indexer-key rows allocated per sequence (tokens, or pools)
    q_seq: np.ndarray     # int32 [n_q]
    q_nvis: np.ndarray    # int32 [n_q], visible cached tokens per query
    cache: np.ndarray     # uint16 [n_seq, T, D]   (bf16 bits)
    idx_k: np.ndarray     # uint16 [n_seq, key_rows, d_idx]
    q: np.ndarray         # uint16 [n_q, n_heads, D]
    idx_q: np.ndarray     # uint16 [n_q, n_idx_heads, d_idx]
    idx_w: np.ndarray     # float32 [n_q, n_idx_heads]
    note: str = ""

    @property
    def n_q(self) -> int:
        return int(self.q_seq.shape[0])

    @property
    def D(self) -> int:
        return self.geom["d_latent"] + self.geom["d_rope"]

    @property
    def max_nvis(self) -> int:
        return int(self.q_nvis.max())


def _fill_normal(out: np.ndarray, cfg_id: int, seq: int, tensor: int,
                 offset: np.ndarray | None = None) -> None:
    """out: uint16 [rows, D] view; rows filled chunk by chunk, in parallel."""
    rows = out.shape[0]
    n_chunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def work(c: int) -> None:
        r0, r1 = c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)
        x = _rng(cfg_id, seq, tensor, c).standard_normal((r1 - r0, out.shape[1]), dtype=np.float32)
        if offset is not None:
            x += offset[None, :]
        out[r0:r1] = f32_to_bf16_bits(x)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(n_chunks)))


def _fill_int(out: np.ndarray, cfg_id: int, seq: int, tensor: int, lo: int, hi: int) -> None:
    rows = out.shape[0]
    n_chunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def work(c: int) -> None:
        r0, r1 = c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)
        v = _rng(cfg_id, seq, tensor, c).integers(lo, hi + 1, size=(r1 - r0, out.shape[1]), dtype=np.int16)
        out[r0:r1] = _INT_BF16[v + 128]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(n_chunks)))


def make_workload(name: str, cfg_id: int, geom: dict, n_seq: int, T: int,
                  q_seq, q_nvis, key_range=(-8, 8), qi_range=(-8, 8),
                  w_range=(1, 4), offset_std: float = 0.0,
                  key_rows: int | None = None, poison_beyond: bool = True,
                  note: str = "") -> Workload:
    """Draw one workload.

    ``q_seq``/``q_nvis`` give each query's sequence and its number of visible
    cached tokens.  Rows a query cannot see because they lie past every
    query's visible range in that sequence are filled with bf16 NaN when
    ``poison_beyond`` is set, so that any read of them shows in the output.
    """
    q_seq = np.asarray(q_seq, dtype=np.int32)
    q_nvis = np.asarray(q_nvis, dtype=np.int32)
    assert q_seq.shape == q_nvis.shape and q_seq.ndim == 1
    kpool = geom["kpool"]
    D = geom["d_latent"] + geom["d_rope"]
    if key_rows is None:
        key_rows = T // kpool if kpool > 1 else T
    n_q = q_seq.shape[0]
    H, HI, DI = geom["n_heads"], geom["n_idx_heads"], geom["d_idx"]

    cache = np.empty((n_seq, T, D), dtype=np.uint16)
    idx_k = np.empty((n_seq, key_rows, DI), dtype=np.uint16)
    for s in range(n_seq):
        off = None
        if offset_std > 0:
            off = (_rng(cfg_id, s, T_OFF).standard_normal(D, dtype=np.float32)
                   * np.float32(offset_std))
        _fill_normal(cache[s], cfg_id, s, T_LATENT, off)
        _fill_int(idx_k[s], cfg_id, s, T_IDXK, *key_range)

    q = np.empty((n_q, H, D), dtype=np.uint16)
    idx_q = np.empty((n_q, HI, DI), dtype=np.uint16)
    idx_w = np.empty((n_q, HI), dtype=np.float32)
    for j in range(n_q):
        q[j] = f32_to_bf16_bits(_rng(cfg_id, j, T_Q).standard_normal((H, D), dtype=np.float32))
        v = _rng(cfg_id, j, T_QI).integers(qi_range[0], qi_range[1] + 1, size=(HI, DI), dtype=np.int16)
        idx_q[j] = _INT_BF16[v + 128]
        idx_w[j] = _rng(cfg_id, j, T_W).integers(w_range[0], w_range[1] + 1, size=HI).astype(np.float32)

    if poison_beyond:
        for s in range(n_seq):
            sel = q_seq == s
            if not sel.any():
                continue
            nv = int(q_nvis[sel].max())
            cache[s, nv:] = BF16_NAN
            idx_k[s, nv // kpool:] = BF16_NAN
    return Workload(name, cfg_id, dict(geom), n_seq, T, key_rows, q_seq, q_nvis,
                    cache, idx_k, q, idx_q, idx_w, note)


# --------------------------------------------------------------------------
# The five problem configurations and the 128K decode metric point.
# --------------------------------------------------------------------------
CONFIGS = ("c0", "c1", "c2", "c3", "c4", "m128k")


def config(name: str, **kw) -> Workload:
    """Full-size workload by name; keyword overrides reach ``make_workload``."""
    if name == "c0":   # tiny decode: B=1, T=4096, k=2048
        return make_workload("c0", 0, GEOM_TOKEN, 1, 4096, [0], [4096], **kw)
    if name == "c1":   # B=8 independent sequences, T=65536 each
        return make_workload("c1", 1, GEOM_TOKEN, 8, 65536, np.arange(8), [65536] * 8, **kw)
    if name == "c2":   # B=4, T=262144, correlated latents, keys in [-4,4] (tie storm)
        return make_workload("c2", 2, GEOM_TOKEN, 4, 262144, np.arange(4), [262144] * 4,
                             key_range=(-4, 4), offset_std=0.5, **kw)
    if name == "c3":   # chunked prefill: 512 consecutive positions at context 131072
        T = 131072
        pos = np.arange(T - 512, T)
        return make_workload("c3", 3, GEOM_TOKEN, 1, T, np.zeros(512), pos + 1, **kw)
    if name == "c4":   # k-pool NoPE, buffer of 2^20 tokens, T-1 cached (tail of 3)
        T = 1 << 20
        return make_workload("c4", 4, GEOM_KPOOL, 1, T, [0], [T - 1], **kw)
    if name == "m128k":  # decode metric point: B=8, T=131072, k=2048
        return decode_128k(8, **kw)
    raise KeyError(name)


def decode_128k(batch: int, **kw) -> Workload:
    """The 128K decode point with ``batch`` sequences (the metric point has
    8); sequence s is drawn from its own streams, so the first 8 sequences
    are the same at every batch size."""
    name = "m128k" if batch == 8 else f"m128k_b{batch}"
    return make_workload(name, 5, GEOM_TOKEN, batch, 131072, np.arange(batch), [131072] * batch, **kw)


def decode_window(batch: int, window: int, T: int = 131072, **kw) -> Workload:
    """Speculative verify: ``batch`` sequences of T cached tokens, each with a
    window of ``window`` query rows at the last positions (row i sees
    T - window + 1 + i tokens), consecutive per sequence."""
    q_seq = np.repeat(np.arange(batch), window)
    q_nvis = np.tile(T - window + 1 + np.arange(window), batch)
    return make_workload(f"win{window}_b{batch}", 6, GEOM_TOKEN, batch, T, q_seq, q_nvis, **kw)


def c3_small(**kw) -> Workload:
    """Prefill variant whose chunk sits at positions 0..511 of a 4096-token
    context, so that early queries keep fewer than top-k candidates."""
    return make_workload("c3s", 13, GEOM_TOKEN, 1, 4096, np.zeros(512), np.arange(512) + 1, **kw)


def indexer_projections(seed: int, n_q: int, n_new: int, n_idx_heads: int = 32, d_idx: int = 128,
                        outliers: int = 4, outlier_scale: float = 16.0):
    """Float32 indexer projections before their preparation: queries
    [n_q, n_idx_heads, d_idx] and keys [n_new, d_idx], standard normal, with
    ``outliers`` channels (the same ones for queries and keys) scaled by
    ``outlier_scale``: the few large channels that make per-element rounding
    uneven, which the rotation spreads out."""
    rng = np.random.default_rng(seed)
    scale = np.ones(d_idx, np.float32)
    scale[rng.permutation(d_idx)[:outliers]] = outlier_scale
    q = rng.standard_normal((n_q, n_idx_heads, d_idx), dtype=np.float32) * scale
    k = rng.standard_normal((n_new, d_idx), dtype=np.float32) * scale
    return q, k
