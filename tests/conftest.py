import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


class _Switches:
    """Sets or clears the library's DG_* tuning switches for one test. The library reads them
    once per process, so every change is followed by a reload; the environment is restored and
    re-read after the test."""

    def __init__(self, mp):
        self._mp = mp

    def setenv(self, var, value):
        self._mp.setenv(var, value)
        _reload_switches()

    def delenv(self, var, raising=True):
        self._mp.delenv(var, raising=raising)
        _reload_switches()


def _reload_switches():
    import moe_grouped_gemm_e4m3_amd as m
    m.reload_tuning_switches()


@pytest.fixture
def switches(monkeypatch):
    yield _Switches(monkeypatch)
    monkeypatch.undo()
    _reload_switches()
