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


@pytest.fixture(scope="session")
def oracle_lib(tmp_path_factory):
    import oracle
    from oracle.build import build, sanitizing
    if sanitizing():  # a sanitizer build of the same source, for this session only
        return oracle.Oracle(build(out=str(tmp_path_factory.mktemp("oracle_asan") / "liboracle.so")))
    return oracle.load()
