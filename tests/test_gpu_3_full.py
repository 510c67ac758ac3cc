"""Parity at the full workload sizes, in the launch configuration the
benchmark times (resident-input plans on the same model budgets).  The 4B
single request is compared on every row of every layer; the packed and
branched workloads on sampled sequences and rows the oracle computes one by
one; the 27B request at its marker row and sampled rows."""
import time

import numpy as np
import pytest

import oracle as O
from s1_workloads import make_batch, make_weights, shape_of
from tests.gpu_util import log, require_gpu
from tests.parity import compare_full_depth, oracle_rows, run_gpu, stack_ref_hidden

pytestmark = pytest.mark.gpu


def test_4b_single_512(gpu_model_4b, oracle_4b, oracle_4b_exact):
    shape = shape_of("4b-single-512")
    b = make_batch("4b-single-512")
    capture = {0: np.arange(512)}
    probs, dec, hid = run_gpu(gpu_model_4b, b, oracle_rows(b, capture), shape.n_layers, shape.d_model)
    t0 = time.time()
    ref = O.prefill_decide(oracle_4b, b, capture=capture)
    log(f"oracle 4b-single-512: {time.time() - t0:.1f} s")
    rx = O.prefill_decide(oracle_4b_exact, b, capture=capture)
    compare_full_depth(b, probs, dec, ref, rx, hid, stack_ref_hidden(ref, capture),
                       stack_ref_hidden(rx, capture), label="4b-single-512")


def test_4b_varlen_16_sampled(gpu_model_4b, oracle_4b, oracle_4b_exact):
    shape = shape_of("4b-varlen-16")
    b = make_batch("4b-varlen-16")
    sample = [9, 4, 15]          # 256, 694 and 826 tokens; 15 is the last in the pack
    rng = np.random.default_rng(3)
    capture = {}
    for i in sample:
        L = int(b.seq_lens[i])
        marks = b.q_marker[b.q_seq == i].tolist()
        capture[i] = np.unique(np.concatenate([marks, rng.choice(L, 24, replace=False), [0, L - 1]]))
    probs, dec, hid = run_gpu(gpu_model_4b, b, oracle_rows(b, capture), shape.n_layers, shape.d_model)
    t0 = time.time()
    ref = O.prefill_decide(oracle_4b, b, capture=capture, seqs=sample)
    log(f"oracle 4b-varlen-16 (3 sequences): {time.time() - t0:.1f} s")
    rx = O.prefill_decide(oracle_4b_exact, b, capture=capture, seqs=sample)
    qs = [j for j in range(b.n_questions) if b.q_seq[j] in sample]
    compare_full_depth(b, probs, dec, ref, rx, hid, stack_ref_hidden(ref, capture),
                       stack_ref_hidden(rx, capture), questions=qs, label="4b-varlen-16 sampled")
    # every question: a probability vector with consistent fields
    for j in range(b.n_questions):
        lo, hi = b.opt_offsets[j], b.opt_offsets[j + 1]
        assert abs(probs[lo:hi].sum() - 1.0) < 1e-5 and (probs[lo:hi] >= 0).all()


def test_4b_branch_4096x20(gpu_model_4b, oracle_4b, oracle_4b_exact):
    shape = shape_of("4b-branch-4096x20")
    b = make_batch("4b-branch-4096x20")
    capture = {0: np.array([0, 1, 2047, 4095])}
    for i in range(1, 21):
        capture[i] = np.array([0, 31, 63])
    probs, dec, hid = run_gpu(gpu_model_4b, b, oracle_rows(b, capture), shape.n_layers, shape.d_model)
    t0 = time.time()
    ref = O.prefill_decide(oracle_4b, b, mode="continuation", capture=capture)
    log(f"oracle 4b-branch-4096x20: {time.time() - t0:.1f} s")
    rx = O.prefill_decide(oracle_4b_exact, b, mode="continuation", capture=capture)
    compare_full_depth(b, probs, dec, ref, rx, hid, stack_ref_hidden(ref, capture),
                       stack_ref_hidden(rx, capture), label="4b-branch-4096x20")


def test_4b_gdn_single_512():
    """The 4B request with Gated DeltaNet linear-attention layers, every row
    of every layer against both oracles under the full-depth gates."""
    import copy
    require_gpu()
    import prefill_only_decision_amd as s1
    shape = shape_of("4b-gdn-single-512")
    b = make_batch("4b-gdn-single-512")
    w = make_weights(shape)
    cfg = s1.make_config(shape, max_tokens=1024, max_seqs=4, max_questions=16, max_options=64,
                         max_prefixes=1, max_positions=1024)
    model = s1.Model(cfg, w.tensors)
    capture = {0: np.arange(512)}
    probs, dec, hid = run_gpu(model, b, oracle_rows(b, capture), shape.n_layers, shape.d_model)
    model.free()
    om = O.OracleModel(shape, w.tensors, dtype=np.float32, keep_decoded=True, act="bf16")
    t0 = time.time()
    ref = O.prefill_decide(om, b, capture=capture)
    log(f"oracle 4b-gdn-single-512: {time.time() - t0:.1f} s")
    ox = copy.copy(om)
    ox.act = "exact"
    rx = O.prefill_decide(ox, b, capture=capture)
    compare_full_depth(b, probs, dec, ref, rx, hid, stack_ref_hidden(ref, capture),
                       stack_ref_hidden(rx, capture), label="4b-gdn-single-512")


@pytest.mark.slow
def test_27b_single_1024():
    require_gpu()
    import prefill_only_decision_amd as s1
    shape = shape_of("27b-single-1024")
    t0 = time.time()
    w = make_weights(shape)
    log(f"27b weights drawn in {time.time() - t0:.1f} s ({w.nbytes() / 1e9:.1f} GB)")
    cfg = s1.make_config(shape, max_tokens=2048, max_seqs=4, max_questions=16, max_options=64,
                         max_prefixes=1, max_positions=2048)
    model = s1.Model(cfg, w.tensors)
    b = make_batch("27b-single-1024")
    rng = np.random.default_rng(5)
    capture = {0: np.unique(np.concatenate([[0, 1023], rng.choice(1024, 14, replace=False)]))}
    probs, dec, hid = run_gpu(model, b, oracle_rows(b, capture), shape.n_layers, shape.d_model)
    model.free()
    t0 = time.time()
    om = O.OracleModel(shape, w.tensors, dtype=np.float32, act="bf16")
    ref = O.prefill_decide(om, b, capture=capture)
    log(f"oracle 27b-single-1024: {time.time() - t0:.1f} s")
    om.act = "exact"
    rx = O.prefill_decide(om, b, capture=capture)
    compare_full_depth(b, probs, dec, ref, rx, hid, stack_ref_hidden(ref, capture),
                       stack_ref_hidden(rx, capture), label="27b-single-1024")
