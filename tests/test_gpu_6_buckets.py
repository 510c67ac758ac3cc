"""Length-bucket plans: one plan (and one captured HIP graph) per length
bucket, refilled with each request that fits (the graph-over-length-buckets
fast path of the Cua-S1 issue's timing comments and RFC #114's plan).  Every
refilled request's answers are held to the float32 oracle under the fixed
gates of tests/parity.py: one request runs layer by layer from the
oracle's inputs through the bucket's graph (1e-2 per layer, its readout
within 1e-2 and no choice flip where the oracle's margin >= 0.02); every
request's end-to-end answers are printed against the oracle.  Under
the row-invariant schedule a refilled bucket also answers bit for bit like a
plan built for the request."""
import numpy as np
import pytest

import oracle as O
from s1_workloads import shape_of
from s1_workloads.batch import random_batch
from tests.gpu_util import log, require_gpu
from tests.parity import decision_gate, layer_local_gate, run_gpu

pytestmark = pytest.mark.gpu

import prefill_only_decision_amd as s1  # noqa: E402

_refs = {}


def _requests(V):
    out = []
    for k, (L, nq) in enumerate([(100, 1), (333, 4), (512, 6), (64, 2), (257, 3)]):
        out.append(random_batch(V, [L], seed=[31, k], questions_per_seq=[nq], choice_range=(2, 10)))
    return out


def _ref(om, k, b):
    if k not in _refs:
        _refs[k] = O.prefill_decide(om, b, capture={0: np.arange(int(b.seq_lens[0]))})
    return _refs[k]


@pytest.mark.parametrize("invariant", [True, False])
def test_bucket_replay_against_oracle(gpu_model_4b, oracle_4b_exact, invariant):
    require_gpu()
    shape = shape_of("4b-single-512")
    V = gpu_model_4b.config.vocab
    bucket = gpu_model_4b.bucket_plan(512, 6, 64)
    for k, b in enumerate(_requests(V)):
        Q = b.n_questions
        bucket.update(b)
        pb, db, _ = run_gpu(gpu_model_4b, b, plan=bucket, invariant=invariant, graph=True)
        ref = _ref(oracle_4b_exact, k, b)
        label = f"bucket 512, request {k} ({int(b.seq_lens[0])} tokens, {Q} questions, invariant={invariant})"
        decision_gate(b, pb, db, ref, None, label=label + " end to end")
        if k == 1:
            L = int(b.seq_lens[0])
            layer_local_gate(gpu_model_4b, b, ref, [0], {0: np.arange(L)}, shape.n_layers, shape.d_model,
                             label=label + " layer-local", invariant=invariant, plan=bucket, graph=True)
        if invariant:
            pf, df, _ = run_gpu(gpu_model_4b, b, invariant=True)
            diff = int((pb.view(np.uint32) != pf.view(np.uint32)).sum())
            log(f"  against a plan built for the request: {diff} probabilities differ")
            assert diff == 0 and np.array_equal(db.view(np.uint8), df.view(np.uint8))
    bucket.free()


def test_bucket_option_slot_holds_placeholders(gpu_model_4b):
    """A bucket with few question slots but a wide option budget, refilled
    with one question over every option slot: the placeholders of the unused
    question slots must fit the device option slot (regression: they once
    overran it into the plan's other tables)."""
    require_gpu()
    V = gpu_model_4b.config.vocab
    bucket = gpu_model_4b.bucket_plan(128, 4, 32)
    from s1_workloads.batch import _assemble
    rng = np.random.default_rng(32)
    toks = rng.integers(0, V, 90).astype(np.int32)
    b = _assemble([toks], [-1], [(0, 89, 0, rng.choice(V, 32, replace=False).astype(np.int32))])
    assert int(b.opt_offsets[-1]) == 32
    bucket.update(b)
    pb, db, _ = run_gpu(gpu_model_4b, b, plan=bucket, invariant=True, graph=False)
    pf, df, _ = run_gpu(gpu_model_4b, b, invariant=True)
    assert np.array_equal(pb.view(np.uint32), pf.view(np.uint32))
    assert np.array_equal(db.view(np.uint8), df.view(np.uint8))
    b2 = random_batch(V, [128], seed=[32, 1], questions_per_seq=[4], choice_range=(2, 2))
    bucket.update(b2)
    p2, d2, _ = run_gpu(gpu_model_4b, b2, plan=bucket, invariant=True, graph=False)
    pf2, df2, _ = run_gpu(gpu_model_4b, b2, invariant=True)
    assert np.array_equal(p2.view(np.uint32), pf2.view(np.uint32))
    bucket.free()


def test_bucket_rejects_what_does_not_fit(gpu_model_4b):
    require_gpu()
    V = gpu_model_4b.config.vocab
    bucket = gpu_model_4b.bucket_plan(256, 2, 16)
    cases = [
        (random_batch(V, [300], seed=1, questions_per_seq=[1]), -4),             # too many tokens
        (random_batch(V, [100], seed=2, questions_per_seq=[3]), -4),             # too many questions
        (random_batch(V, [100, 50], seed=3, questions_per_seq=[1, 1]), -1),     # two sequences
        (random_batch(V, [100], seed=4, questions_per_seq=[2], choice_range=(9, 9)), -4),  # options
    ]
    for b, code in cases:
        if code == -4 and int(b.opt_offsets[-1]) <= 16 and b.n_questions <= 2 and int(b.seq_lens.max()) <= 256:
            continue    # the seeded draw happened to fit
        with pytest.raises(s1.S1Error) as e:
            bucket.update(b)
        assert e.value.code == code, (e.value.code, code)
    plain = gpu_model_4b.plan(random_batch(V, [50], seed=5))
    with pytest.raises(s1.S1Error) as e:
        plain.update(random_batch(V, [50], seed=6))
    assert e.value.code == -1
    plain.free()
    bucket.free()
