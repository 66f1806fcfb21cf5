"""Host-only checks of the C ABI library (no GPU needed): it loads, exports
every function that include/dsa.h declares, answers the host-only queries,
and refuses to run without a gfx950 device rather than falling back."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dsa_index_scores", "dsa_topk", "dsa_mla_attend", "dsa_decode_step", "dsa_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from deepseek_sparse_attention_amd import binding as B
    lib = ctypes.CDLL(B._LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(B.EXPORTS) == set(declared_functions())


def test_host_queries():
    from deepseek_sparse_attention_amd import binding as B
    from deepseek_sparse_attention_amd import inputs as I
    assert B._lib.dsa_status_str(0) == b"ok"
    assert B._lib.dsa_status_str(-3).startswith(b"workspace")
    n = B.workspace_bytes(I.GEOM_TOKEN, 8, 131072)
    assert n > 8 * 131072 * 4          # holds at least the score matrix
    assert B.workspace_bytes(I.GEOM_TOKEN, 0, 100) == 0
    bad = dict(I.GEOM_TOKEN, n_heads=32)
    assert B.workspace_bytes(bad, 1, 100) == 0
    assert B.workspace_bytes(dict(I.GEOM_TOKEN, top_k=4097), 1, 100) == 0
    assert B.workspace_bytes(dict(I.GEOM_KPOOL, top_k=2050), 1, 100) == 0


def test_no_device_means_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from deepseek_sparse_attention_amd import binding as B
    assert B._lib.dsa_device_check() == B.DSA_ERR_DEVICE
    with pytest.raises(B.DSAError):
        B.device_check()


@pytest.mark.parametrize("geom_name", ["token", "kpool"])
def test_workspace_sizes_leave_room_for_the_histogram_region(geom_name):
    """The histogram region is the workspace's first sixteenth, in whole
    20 KiB blocks: every size the library asks for must hold the call's
    n_q blocks there."""
    from deepseek_sparse_attention_amd import binding as B
    from deepseek_sparse_attention_amd import inputs as I
    g = I.GEOM_TOKEN if geom_name == "token" else I.GEOM_KPOOL
    for n_q in (1, 2, 3, 8, 37, 64, 200, 4096):
        for m in (1, 100, 2047, 2052, 4096, 16384, 16385, 131072, 1 << 20):
            n = B.workspace_bytes(g, n_q, m)
            assert n % 256 == 0
            assert (n // 16) // 20480 >= n_q, (n_q, m, n)
