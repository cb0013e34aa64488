import json
import os
import sys

import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")

# The suite loads the in-tree library.  It rebuilds it when nothing is built or
# when the sources changed since the last build (the hash the build records
# beside the library differs), so a stale library is never tested.
import importlib.util as _ilu   # the package itself refuses to import unbuilt

_spec = _ilu.spec_from_file_location(
    "_moe_build", os.path.join(ROOT, "mixture_experts_expert_amd", "build.py"))
_build = _ilu.module_from_spec(_spec)
_spec.loader.exec_module(_build)
if _build.is_stale():
    print("conftest: libmoe_native.so is missing or older than its sources; rebuilding", flush=True)
    _build.build(verbose=True)


@pytest.hookimpl(tryfirst=True)
def pytest_configure(config):
    # A test stuck in a device call ends after 600 s with its name, instead
    # of holding the whole run, unless the command line sets a timeout.
    if hasattr(config.option, "timeout") and not config.option.timeout:
        config.option.timeout = 600.0
        config.option.timeout_method = "thread"
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes on the CPU side")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def skew_alpha():
    return load_golden("skew_alpha.json")["alpha"]
