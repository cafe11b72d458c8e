import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


import pytest  # noqa: E402


@pytest.fixture
def lib_options():
    """Setter of the library's process-wide launch options (tp_set_options);
    the options in force before the test are restored after it."""
    from attention_column_gemm_amd import binding as B
    saved = B.tp_get_options()

    def set_options(tile=None, split_tail=None):
        cur = B.tp_get_options()
        B.tp_set_options(cur[0] if tile is None else tile, cur[1] if split_tail is None else split_tail)

    yield set_options
    B.tp_set_options(*saved)
