"""Whole-model parity through the C ABI on small shapes: the tiny fp32 hybrid,
and a reduced-depth bf16 hybrid with the 4B head dimensions (128), covering
varlen packing, ragged tails, branches from a prefix, empty requests, and the
invariances of RFC #114 section 6 (reordering, repeated requests).  The
reference is the float64 oracle without activation rounding; the gates are
those of tests/parity.py (RFC #114 section 6): every layer within 1e-2
relative L2 when run from the oracle's input to it, probabilities within
1e-2 end to end, no choice flip where the oracle's margin >= 0.02."""
from dataclasses import replace

import numpy as np
import pytest

import oracle as O
from s1_workloads import make_batch, make_weights, shape_of
from s1_workloads.batch import random_batch
from tests.gpu_util import log, require_gpu
from tests.parity import (HIDDEN_TOL, PROB_TOL, decision_gate, end_to_end_drift, layer_local_gate, oracle_rows,
                          ref_rows, run_gpu)

pytestmark = pytest.mark.gpu

import prefill_only_decision_amd as s1  # noqa: E402

MINI = replace(shape_of("4b-single-512"), name="bf16-mini", n_layers=4, d_model=512, ffn=1024,
               vocab=4096, la_heads=4, fa_q_heads=4, fa_kv_heads=2, shape_id=77)

MINI_GDN = replace(MINI, name="bf16-mini-gdn", la_kind="gdn", shape_id=78)

_models = {}


def _model(shape):
    """(GPU model, float64 oracle without activation rounding)."""
    require_gpu()
    if shape.name not in _models:
        w = make_weights(shape)
        cfg = s1.make_config(shape, max_tokens=4096, max_seqs=16, max_questions=64, max_options=64,
                             max_prefixes=2, max_positions=4096)
        _models[shape.name] = (s1.Model(cfg, w.tensors), O.OracleModel(shape, w.tensors))
    return _models[shape.name]


def _full_check(shape, batch, label, mode="plain"):
    """End-to-end decisions and per-layer drift (reported) from one run, then
    the layer-local gate at every layer over every row."""
    model, om = _model(shape)
    seqs = [i for i in range(batch.n_seqs) if batch.seq_lens[i] > 0]
    cap = {i: np.arange(int(batch.seq_lens[i])) for i in seqs}
    probs, dec, hid = run_gpu(model, batch, oracle_rows(batch, cap), shape.n_layers, shape.d_model)
    ref = O.prefill_decide(om, batch, mode=mode, capture=cap)
    drift = end_to_end_drift(hid, ref_rows(ref, cap))
    log(f"{label}: end-to-end rel L2 per layer " + " ".join(f"{x:.1e}" for x in drift))
    if shape.dtype == "f32":    # fp32 path: end to end within the per-layer gate too
        assert max(drift) <= HIDDEN_TOL
    out = decision_gate(batch, probs, dec, ref, PROB_TOL, label=label)
    if seqs:
        # a branch's captured rows are its own rows in both oracle modes (the
        # plain mode runs prefix + branch and returns the rows past the prefix)
        layer_local_gate(model, batch, ref, seqs, cap, shape.n_layers, shape.d_model, label=label)
    return out


def test_tiny_workload():
    _full_check(shape_of("tiny-fp32"), make_batch("tiny-fp32"), "tiny-fp32 workload")


def test_tiny_varlen_and_branches():
    b = random_batch(4096, [70, 1, 130, 64, 0, 33], seed=4, prefix_of=[-1, -1, -1, 0, -1, 0],
                     questions_per_seq=[0, 1, 3, 2, 0, 1])
    _full_check(shape_of("tiny-fp32"), b, "tiny varlen+branches")


def test_bf16_mini_varlen_ragged():
    b = random_batch(MINI.vocab, [300, 1, 130, 64, 257], seed=8, questions_per_seq=[4, 1, 2, 1, 3])
    _full_check(MINI, b, "bf16-mini varlen")


def test_bf16_mini_branches():
    # prefix of 100 (not a multiple of the scan chunk), branches of 64, 1, 65
    b = random_batch(MINI.vocab, [100, 64, 1, 65, 40], seed=9, prefix_of=[-1, 0, 0, 0, -1],
                     questions_per_seq=[0, 2, 1, 2, 1])
    _full_check(MINI, b, "bf16-mini branches")


def test_gdn_mini_varlen_ragged():
    # Gated DeltaNet layers (short convolution, L2-normalised q/k, delta rule)
    b = random_batch(MINI_GDN.vocab, [300, 1, 130, 64, 257, 2], seed=18, questions_per_seq=[4, 1, 2, 1, 3, 1])
    _full_check(MINI_GDN, b, "bf16-mini GDN varlen")


def test_gdn_mini_branches():
    # branches continue from the prefix's state and last three pre-convolution
    # rows; prefixes of 100 and 2 tokens (shorter than the convolution)
    b = random_batch(MINI_GDN.vocab, [100, 64, 1, 65, 2, 40, 3], seed=19, prefix_of=[-1, 0, 0, 0, -1, 4, 4],
                     questions_per_seq=[0, 2, 1, 2, 0, 1, 1])
    _full_check(MINI_GDN, b, "bf16-mini GDN branches")
    _full_check(MINI_GDN, b, "bf16-mini GDN branches (continuation oracle)", mode="continuation")


def test_empty_request():
    model, _ = _model(MINI)
    b = random_batch(MINI.vocab, [], seed=1)
    probs, dec, _ = run_gpu(model, b)
    assert probs.size == 0 and dec.size == 0
    b = random_batch(MINI.vocab, [12, 0], seed=1, questions_per_seq=[0, 0])
    probs, dec, _ = run_gpu(model, b)
    assert dec.size == 0


def test_repeated_requests_are_bitwise_identical():
    model, _ = _model(MINI)
    b = random_batch(MINI.vocab, [200, 64, 9], seed=12, prefix_of=[-1, 0, -1])
    rows = list(range(0, 273, 7))
    outs = [run_gpu(model, b, rows, MINI.n_layers, MINI.d_model) for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0])
        assert np.array_equal(o[1], outs[0][1])
        assert np.array_equal(o[2], outs[0][2])


def test_host_path_equals_plan_path():
    model, _ = _model(MINI)
    b = random_batch(MINI.vocab, [150, 31], seed=13)
    p1, d1, _ = run_gpu(model, b)
    p2, d2, t = model.decide(b)
    assert np.array_equal(p1, p2) and np.array_equal(d1, d2)
    assert t["tokens"] == 181


def test_host_path_replays_repeated_structures():
    """The boundary call replays a captured HIP graph when a batch repeats
    the previous call's structure (lengths, prefixes, questions, markers,
    option counts) with new token and option ids: every call must answer
    like a plan built for its batch, and another structure in between must
    not reuse the graph."""
    model, _ = _model(MINI)
    base = random_batch(MINI.vocab, [150, 31, 20], seed=15, prefix_of=[-1, 0, -1])
    other = random_batch(MINI.vocab, [90, 40], seed=16)
    rng = np.random.default_rng(17)

    def refill(b):
        opt = np.concatenate([rng.choice(MINI.vocab, int(b.opt_offsets[j + 1] - b.opt_offsets[j]), replace=False)
                              for j in range(b.n_questions)]).astype(np.int32)
        return replace(b, token_ids=rng.integers(0, MINI.vocab, b.token_ids.shape[0]).astype(np.int32),
                       opt_ids=opt)

    for k, b in enumerate([base, refill(base), refill(base), other, refill(base), refill(base)]):
        p1, d1, _ = run_gpu(model, b)
        p2, d2, _ = model.decide(b)
        log(f"call {k}: {int((p1 != p2).sum())} probabilities differ from a plan of the batch")
        assert np.array_equal(p1, p2) and np.array_equal(d1, d2), k


def test_option_and_question_permutation():
    model, _ = _model(MINI)
    b = random_batch(MINI.vocab, [180, 77], seed=14, questions_per_seq=[3, 2])
    p, d, _ = run_gpu(model, b)
    rng = np.random.default_rng(0)
    # permute each question's options (noul keeps its [yes, no] meaning: skip)
    b2 = random_batch(MINI.vocab, [180, 77], seed=14, questions_per_seq=[3, 2])
    perms = []
    for j in range(b.n_questions):
        lo, hi = b.opt_offsets[j], b.opt_offsets[j + 1]
        pm = rng.permutation(hi - lo) if b.q_type[j] != 2 else np.arange(hi - lo)
        b2.opt_ids[lo:hi] = b.opt_ids[lo:hi][pm]
        perms.append(pm)
    p2, _, _ = run_gpu(model, b2)
    for j in range(b.n_questions):
        lo, hi = b.opt_offsets[j], b.opt_offsets[j + 1]
        np.testing.assert_allclose(p2[lo:hi], p[lo:hi][perms[j]], rtol=1e-5, atol=1e-7)
    # reverse the question order
    order = np.arange(b.n_questions)[::-1]
    b3 = random_batch(MINI.vocab, [180, 77], seed=14, questions_per_seq=[3, 2])
    ks = np.diff(b.opt_offsets)[order]
    b3.q_seq, b3.q_marker, b3.q_type = b.q_seq[order], b.q_marker[order], b.q_type[order]
    b3.opt_offsets = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    b3.opt_ids = np.concatenate([b.options_of(j) for j in order]).astype(np.int32)
    p3, d3, _ = run_gpu(model, b3)
    for jj, j in enumerate(order):
        np.testing.assert_array_equal(p3[b3.opt_offsets[jj]:b3.opt_offsets[jj + 1]], p[b.opt_offsets[j]:b.opt_offsets[j + 1]])
        assert d3[jj] == d[j]


def test_branch_matches_plain_forward_on_gpu():
    """A branch of a prefix answers like the plain sequence prefix + branch
    (RFC #114 plan comment: a continuation equals the plain forward up to
    rounding); rounding differs (other chunk and tile boundaries)."""
    model, _ = _model(MINI)
    b = random_batch(MINI.vocab, [130, 70], seed=15, prefix_of=[-1, 0], questions_per_seq=[0, 3])
    p, d, _ = run_gpu(model, b)
    plain = random_batch(MINI.vocab, [200], seed=16, questions_per_seq=[1])
    plain.token_ids = np.concatenate([b.tokens_of(0), b.tokens_of(1)]).astype(np.int32)
    plain.q_seq = np.zeros(3, np.int32)
    plain.q_marker = (b.q_marker + 130).astype(np.int32)
    plain.q_type, plain.opt_offsets, plain.opt_ids = b.q_type, b.opt_offsets, b.opt_ids
    p2, _, _ = run_gpu(model, plain)
    log(f"branch vs plain: max|dp| {np.abs(p - p2).max():.2e}")
    assert np.abs(p - p2).max() < 2e-3


def test_varlen_matches_each_request_alone():
    model, _ = _model(MINI)
    b = random_batch(MINI.vocab, [190, 65, 300], seed=17, questions_per_seq=[2, 1, 2])
    p, _, _ = run_gpu(model, b)
    for i in range(3):
        qs = np.nonzero(b.q_seq == i)[0]
        alone = random_batch(MINI.vocab, [int(b.seq_lens[i])], seed=18, questions_per_seq=[1])
        alone.token_ids = b.tokens_of(i).astype(np.int32)
        alone.q_seq = np.zeros(len(qs), np.int32)
        alone.q_marker, alone.q_type = b.q_marker[qs], b.q_type[qs]
        ks = np.diff(b.opt_offsets)[qs]
        alone.opt_offsets = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
        alone.opt_ids = np.concatenate([b.options_of(j) for j in qs]).astype(np.int32)
        pa, _, _ = run_gpu(model, alone)
        ref = np.concatenate([p[b.opt_offsets[j]:b.opt_offsets[j + 1]] for j in qs])
        assert np.abs(pa - ref).max() < 2e-3


def test_graph_replay_matches_eager():
    """Every replay of the captured plan equals the eager run bit for bit,
    with eager work and synchronisations between replays; changing the
    output buffers re-captures."""
    import torch
    from tests.gpu_util import stream_ptr
    model, _ = _model(MINI)
    b = random_batch(MINI.vocab, [200, 64, 9, 130], seed=19, prefix_of=[-1, 0, -1, -1])
    p_ref, d_ref, _ = run_gpu(model, b)
    plan = model.plan(b)
    plan.set_graph(True)
    stream = torch.cuda.Stream()
    for rep in range(4):
        dp = torch.full((plan.n_options,), -1.0, dtype=torch.float32, device="cuda")
        dd = torch.zeros((plan.n_questions, 6), dtype=torch.float32, device="cuda")
        if rep == 3:   # other output buffers: a new capture
            dp, dd = dp.clone(), dd.clone()
        with torch.cuda.stream(stream):
            plan.run(dp.data_ptr(), dd.data_ptr(), stream.cuda_stream)
        torch.cuda.synchronize()
        got = dp.cpu().numpy()
        assert np.array_equal(got, p_ref), rep
        dec = dd.cpu().numpy().copy().view(np.uint8).view(s1.DECISION_DTYPE).reshape(-1)
        assert np.array_equal(dec, d_ref), rep
        run_gpu(model, random_batch(MINI.vocab, [50], seed=rep))   # eager work in between
    plan.free()
