"""Failure paths forced from the host (no kernel faults, nothing hangs): an
allocation failure injected at every allocation of a model load, of a plan,
of a capture and of the boundary call (the S1_TEST_FAIL_ALLOC hook makes the
n-th allocation fail as if the device were out of memory).  Each call must
return S1_ENOMEM, leave no device memory behind, and leave the model usable:
RFC #114 section 2 (explicit errors; resource ownership kept until device
work finishes, error paths included)."""
import os

import numpy as np
import pytest

from s1_workloads import make_batch, make_weights, shape_of
from tests.gpu_util import log, require_gpu

pytestmark = pytest.mark.gpu

HOOK = "S1_TEST_FAIL_ALLOC"
_tag = [0]


def _with_failure(n, fn):
    # the count restarts whenever the variable's text changes: a fresh tag
    # per call makes "the n-th allocation of this call" unambiguous
    _tag[0] += 1
    os.environ[HOOK] = f"{n}@{_tag[0]}"
    try:
        return fn()
    finally:
        del os.environ[HOOK]


def test_load_fails_cleanly_at_every_allocation():
    torch = require_gpu()
    import prefill_only_decision_amd as s1
    shape = shape_of("tiny-fp32")
    w = make_weights(shape)
    cfg = s1.make_config(shape, max_tokens=1024)
    # one whole load first: the library's code object, its streams and the
    # runtime's own pools are in place before the count starts
    warm = s1.Model(cfg, w.tensors)
    warm.decide(make_batch("tiny-fp32"))
    warm.free()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    failed = 0
    for n in range(1, 400):
        try:
            m = _with_failure(n, lambda: s1.Model(cfg, w.tensors))
        except s1.S1Error as e:
            assert e.code == s1.binding.S1_ENOMEM, (n, e.code, str(e))
            failed += 1
            continue
        m.free()       # n is past the last allocation of a load
        break
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    log(f"load: {failed} allocations, each failed in turn with S1_ENOMEM; device memory "
        f"{(free0 - free1) / 2**20:.1f} MiB lower afterwards")
    assert failed >= 10
    assert free0 - free1 < 16 * 2**20


def test_model_stays_usable_after_failed_calls():
    torch = require_gpu()
    import prefill_only_decision_amd as s1
    shape = shape_of("tiny-fp32")
    w = make_weights(shape)
    m = s1.Model(s1.make_config(shape, max_tokens=1024), w.tensors)
    b = make_batch("tiny-fp32")
    # the first boundary call allocates the model's request block: make it fail
    with pytest.raises(s1.S1Error) as e:
        _with_failure(1, lambda: m.decide(b))
    assert e.value.code == s1.binding.S1_ENOMEM
    p_ok, d_ok, _ = m.decide(b)
    p_again, d_again, _ = m.decide(b)
    assert np.array_equal(p_ok, p_again) and np.array_equal(d_ok, d_again)
    # plan creation, capture and layer inputs
    with pytest.raises(s1.S1Error) as e:
        _with_failure(1, lambda: m.plan(b))
    assert e.value.code == s1.binding.S1_ENOMEM
    plan = m.plan(b)
    hid = torch.zeros((shape.n_layers + 1, 4, shape.d_model), dtype=torch.float32, device="cuda")
    with pytest.raises(s1.S1Error) as e:
        _with_failure(1, lambda: plan.set_capture(np.arange(4), hid.data_ptr()))
    assert e.value.code == s1.binding.S1_ENOMEM
    with pytest.raises(s1.S1Error) as e:
        _with_failure(1, lambda: plan.set_layer_inputs(np.arange(4), hid.data_ptr()))
    assert e.value.code == s1.binding.S1_ENOMEM
    dp = torch.zeros(plan.n_options, dtype=torch.float32, device="cuda")
    dd = torch.zeros((plan.n_questions, 6), dtype=torch.float32, device="cuda")
    plan.run(dp.data_ptr(), dd.data_ptr())
    torch.cuda.synchronize()
    assert np.array_equal(dp.cpu().numpy(), p_ok)
    plan.free()
    m.free()
    log("boundary call, plan, capture and layer inputs: S1_ENOMEM, then the same model answers as before")
