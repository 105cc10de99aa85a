import ctypes
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _keep_freed_memory():
    """Let glibc reuse freed memory instead of returning it to the system.

    The oracle builds float64 temporaries of up to a few hundred MB per query
    row; with the default policy each is a fresh mapping whose first touch
    page-faults (measured here: ~3 s of a 3.5 s oracle row at 65,536 tokens,
    0.7 s once the memory is reused). M_MMAP_MAX = 0 keeps large blocks on
    the heap and M_TRIM_THRESHOLD = 16 GiB keeps the freed heap mapped.
    """
    try:
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-4, 0)          # M_MMAP_MAX
        libc.mallopt(-1, 1 << 34)    # M_TRIM_THRESHOLD
    except OSError:
        pass


_keep_freed_memory()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes on the CPU oracle)")
