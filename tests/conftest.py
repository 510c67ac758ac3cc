import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of CPU oracle time)")


# ---------------------------------------------------------------- GPU tier
# Session-wide weights and models for the full-size workloads: drawing the
# 4B weights takes seconds, loading them a few more, so every GPU test that
# uses the 4B shape shares one copy.
_cache = {}


def _get(key, make):
    if key not in _cache:
        _cache[key] = make()
    return _cache[key]


@pytest.fixture(scope="session")
def weights_4b():
    from s1_workloads import make_weights, shape_of
    return _get("w4b", lambda: make_weights(shape_of("4b-single-512")))


@pytest.fixture(scope="session")
def gpu_model_4b(weights_4b):
    from tests.gpu_util import require_gpu
    require_gpu()
    import prefill_only_decision_amd as s1
    from s1_workloads import shape_of

    def make():
        cfg = s1.make_config(shape_of("4b-single-512"), max_tokens=32768, max_seqs=64,
                             max_questions=256, max_options=256, max_prefixes=4,
                             max_positions=8192)
        return s1.Model(cfg, weights_4b.tensors)
    return _get("m4b", make)


@pytest.fixture(scope="session")
def oracle_4b_exact(weights_4b):
    """The float32 oracle of the 4B shape without activation rounding."""
    import numpy as np
    import oracle
    from s1_workloads import shape_of
    return _get("o4bx", lambda: oracle.OracleModel(shape_of("4b-single-512"), weights_4b.tensors,
                                                    dtype=np.float32, keep_decoded=True))
