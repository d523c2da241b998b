import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    """The oracle package; RT_ORACLE_DIR may point at a modified copy (used by
    tests/test_oracle_mutants.py to show that the pins catch planted errors)."""
    alt = os.environ.get("RT_ORACLE_DIR")
    if alt:
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "oracle_under_test", os.path.join(alt, "__init__.py"),
            submodule_search_locations=[alt])
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(force=True)
        return mod
    import oracle
    oracle.build()
    return oracle
