import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture
def tune(monkeypatch):
    """Kernel-variant overrides for every plan a test creates: ``tune(cu=2,
    cu_pd=1)`` makes each ConvBnSilu built afterwards (in this test) pass
    those keys to tg_conv_bn_silu_create_tuned, merged under any tuning the
    call gives itself. Values of None or "" are skipped (the kernel's
    default)."""
    from conv2d_batchnorm_silu_amd import binding as B
    over = {}
    orig = B.ConvBnSilu.__init__

    def init(self, *args, tuning=None, **kw):
        merged = dict(over)
        if isinstance(tuning, dict):
            merged.update(tuning)
        elif tuning is not None:
            raise TypeError("tests pass tuning as a dict")
        orig(self, *args, tuning=merged or None, **kw)

    monkeypatch.setattr(B.ConvBnSilu, "__init__", init)

    def set_(**kv):
        for k, v in kv.items():
            if v is None or v == "":
                over.pop(k, None)
            else:
                over[k] = int(v)
    return set_
