import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import oracle_pool  # noqa: E402


def _gpu_session(config) -> bool:
    """GPU tests may run: a GPU is present and the marker expression does not exclude them."""
    expr = (config.getoption("markexpr") or "").replace(" ", "")
    return os.path.exists("/dev/kfd") and "notgpu" not in expr and os.environ.get("KVQ_ORACLE_POOL", "1") != "0"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # the oracle workers start now, before any test touches the GPU
    if _gpu_session(config):
        oracle_pool.start()


def pytest_collection_finish(session):
    jobs = {}
    for item in session.items:
        mod_jobs = getattr(item.module, "ORACLE_JOBS", None)
        if mod_jobs and item.get_closest_marker("gpu") is not None:
            for key in getattr(item.function, "oracle_jobs", ()):
                jobs[key] = mod_jobs[key]
    oracle_pool.submit(jobs)


def pytest_unconfigure(config):
    oracle_pool.stop()
