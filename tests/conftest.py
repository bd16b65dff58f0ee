import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# the two decode batches, generated once per session (host arrays)
@pytest.fixture(scope="session")
def c3():
    import synth
    return synth.c3()


@pytest.fixture(scope="session")
def c4():
    import synth
    return synth.c4()
