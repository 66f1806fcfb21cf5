"""Host-side checks of bench.py that need no GPU: the helpers it uses to tie
committed counter readings to the kernel source still find that source."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_score_kernel_hash_finds_the_kernel():
    h = _bench().score_kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
