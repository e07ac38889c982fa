import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# A fresh checkout holds no built library (it is not versioned): build it
# once before any test imports the binding, which refuses to run without it.
if not os.path.exists(os.path.join(ROOT, "decode_step_attention_amd", "libftm.so")):
    from decode_step_attention_amd import build as _build
    _build.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture
def tuning(monkeypatch):
    """Sets FTM_* tuning variables for one test.  The library reads them once,
    so every change is followed by ftm_tuning_reload, and so is the restore."""
    from decode_step_attention_amd import ftm

    class Tuning:
        def set(self, name, value):
            monkeypatch.setenv(name, str(value))
            ftm.ftm_tuning_reload()

    yield Tuning()
    monkeypatch.undo()
    ftm.ftm_tuning_reload()
