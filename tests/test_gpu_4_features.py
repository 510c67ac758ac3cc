"""Full-vocabulary log-probability features on the GPU against the oracle:
the vocabulary log-sum-exp kernel and the whole feature computation through
their C-ABI entry points on seeded inputs (full 4B vocabulary and width,
ragged vocabulary sizes, fp32 models), and the plan-level features of a whole
request against the oracle's forward.

Tolerance.  The bf16 path forms each logit on MFMA from the normalised row
split into bf16 hi + lo (|h - hi - lo| <= 2^-17 |h|) with fp32 accumulation,
then exp / log in fp32.  For logits of size |z| <= 50 and d <= 5120 that
gives errors of order 1e-5 on lse; the gate is 2e-4 absolute on lse and logp
(1e-3 at the large-logit scale), four orders tighter than the 1e-2 the
probabilities are held to."""
import numpy as np
import pytest

import oracle as O
from s1_workloads import f32_to_bf16_bits, make_batch, make_weights, shape_of
from tests.gpu_util import dev, dev_bits, log, require_gpu, stream_ptr

pytestmark = pytest.mark.gpu

import prefill_only_decision_amd as s1  # noqa: E402
from prefill_only_decision_amd import binding as B  # noqa: E402


def _embed_bits(rng, V, d, std):
    return f32_to_bf16_bits(rng.standard_normal((V, d), dtype=np.float32) * np.float32(std))


def _rows(rng, n, d):
    return (rng.standard_normal((n, d)) * rng.uniform(0.5, 3.0, (n, 1))).astype(np.float32)


@pytest.mark.parametrize("V,d,R,std", [
    (151936, 2560, 3, 0.02),      # the 4B vocabulary and width, three marker rows
    (151936, 2560, 40, 0.02),     # one 64-row launch
    (151936, 2560, 70, 0.02),     # a 64-row and a 32-row launch
    (151936, 5120, 5, 0.02),      # the 27B width
    (1000, 256, 7, 0.2),          # ragged vocabulary tail, large logits
    (129, 128, 33, 0.5),          # one row in the last block, one k chunk
    (1, 128, 2, 0.5),             # a vocabulary of one token: lse = z
    # k-chunk counts that leave every remainder of the four-deep load ring
    (5000, 256, 5, 0.02),         # 32-row pass, 2 chunks of 128
    (5000, 384, 3, 0.02),         # 3 chunks
    (5000, 384, 40, 0.02),        # 64-row pass, 6 chunks of 64
    (5000, 640, 70, 0.02),        # 64-row pass (10 chunks) and 32-row pass (5)
    (5000, 2688, 9, 0.02),        # 21 chunks
])
def test_vocab_lse_bf16(V, d, R, std):
    torch = require_gpu()
    log(f"vocab lse bf16 V={V} d={d} R={R} std={std}")
    rng = np.random.default_rng([V, d, R])
    E = _embed_bits(rng, V, d, std)
    n_x = R + 5
    x = _rows(rng, n_x, d)
    w = rng.uniform(0.5, 1.5, d).astype(np.float32)
    rows = rng.choice(n_x, R, replace=False).astype(np.int32)
    dl = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    dE, dx, dw, dr = dev_bits(E), dev(x), dev(w), dev(rows)
    B.vocab_lse(B.S1_BF16, dx.data_ptr(), d, dw.data_ptr(), 1e-6, dE.data_ptr(), V, R, dr.data_ptr(),
                dl.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    got = dl.cpu().numpy()
    _, ref = O.vocab_log_probs(x[rows], w, E, 1e-6, [0], [0])
    tol = 2e-4 if std <= 0.02 else 1e-3
    err = np.abs(got - ref).max()
    log(f"  max |d lse| {err:.2e} (lse {ref.min():.2f} .. {ref.max():.2f})")
    assert np.isfinite(got).all() and err <= tol, err


def test_vocab_lse_f32():
    torch = require_gpu()
    rng = np.random.default_rng(11)
    V, d, R = 4096, 256, 9
    E = (rng.standard_normal((V, d)) * 0.3).astype(np.float32)
    x = _rows(rng, R, d)
    w = rng.uniform(0.5, 1.5, d).astype(np.float32)
    rows = np.arange(R, dtype=np.int32)[::-1].copy()
    dl = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    dE, dx, dw, dr = dev(E), dev(x), dev(w), dev(rows)
    B.vocab_lse(B.S1_F32, dx.data_ptr(), d, dw.data_ptr(), 1e-6, dE.data_ptr(), V, R, dr.data_ptr(),
                dl.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    _, ref = O.vocab_log_probs(x[rows], w, E, 1e-6, [0], [0])
    assert np.abs(dl.cpu().numpy() - ref).max() <= 1e-4


def _feature_case(rng, n_rows, V, n_groups):
    """Targets over n_rows rows (rows repeat), candidates of 0..4 targets in
    groups; some targets belong to no candidate."""
    rows, toks, cand_off, cand_group = [], [], [0], []
    for g in range(n_groups):
        for _ in range(int(rng.integers(1, 6))):
            k = int(rng.integers(0, 5))
            base = int(rng.integers(0, n_rows))
            for i in range(k):
                rows.append(min(base + i, n_rows - 1))
                toks.append(int(rng.integers(0, V)))
            cand_off.append(len(rows))
            cand_group.append(100 - 7 * g)      # group ids need not be small or sorted
    for _ in range(3):                            # targets outside every candidate
        rows.append(int(rng.integers(0, n_rows)))
        toks.append(int(rng.integers(0, V)))
    perm = rng.permutation(len(cand_group))       # candidates of a group interleave
    return (np.array(rows, np.int32), np.array(toks, np.int32), np.array(cand_off, np.int32),
            np.array(cand_group, np.int32), perm)


@pytest.mark.parametrize("dtype,V,d,n_rows,n_groups", [
    ("bf16", 151936, 2560, 48, 9),
    ("bf16", 1000, 256, 5, 3),
    ("f32", 4096, 256, 20, 6),
])
def test_token_logprobs(dtype, V, d, n_rows, n_groups):
    torch = require_gpu()
    log(f"token logprobs {dtype} V={V} d={d} rows={n_rows} groups={n_groups}")
    rng = np.random.default_rng([V, d, n_rows])
    bf = dtype == "bf16"
    E = _embed_bits(rng, V, d, 0.02) if bf else (rng.standard_normal((V, d)) * 0.3).astype(np.float32)
    x = _rows(rng, n_rows, d)
    w = rng.uniform(0.5, 1.5, d).astype(np.float32)
    rows, toks, off, grp, _ = _feature_case(rng, n_rows, V, n_groups)
    C = len(grp)
    n = len(rows)
    dlp = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    dcl = torch.full((C,), float("nan"), dtype=torch.float32, device="cuda")
    dcn = torch.full((C,), float("nan"), dtype=torch.float32, device="cuda")
    dE = dev_bits(E) if bf else dev(E)
    dx, dw = dev(x), dev(w)
    B.token_logprobs(B.S1_BF16 if bf else B.S1_F32, dx.data_ptr(), n_rows, d, dw.data_ptr(), 1e-6,
                     dE.data_ptr(), V, rows, toks, off, grp, dlp.data_ptr(), dcl.data_ptr(), dcn.data_ptr(),
                     stream_ptr())
    torch.cuda.synchronize()
    ref_lp, _ = O.vocab_log_probs(x, w, E, 1e-6, rows, toks)
    ref_cl, ref_cn = O.candidate_log_probs(ref_lp, off, grp)
    lp, cl, cn = dlp.cpu().numpy(), dcl.cpu().numpy(), dcn.cpu().numpy()
    e1 = np.abs(lp - ref_lp).max()
    e2 = np.abs(cl - ref_cl).max()
    e3 = np.abs(cn - ref_cn).max()
    log(f"  max |d logp| {e1:.2e}, |d cand| {e2:.2e}, |d norm| {e3:.2e}")
    assert e1 <= 2e-4
    # a candidate sums at most 4 targets; its normalisation subtracts a log-sum-exp of such sums
    assert e2 <= 8e-4 and e3 <= 1.6e-3
    for g in np.unique(grp):
        assert abs(np.exp(cn[grp == g]).sum() - 1.0) < 1e-4


def test_token_logprobs_run_twice_is_identical():
    """The merge order is fixed: two runs give the same bits."""
    torch = require_gpu()
    rng = np.random.default_rng(5)
    V, d = 151936, 2560
    E = _embed_bits(rng, V, d, 0.02)
    x = _rows(rng, 8, d)
    w = np.ones(d, np.float32)
    rows, toks, off, grp, _ = _feature_case(rng, 8, V, 3)
    dE, dx, dw = dev_bits(E), dev(x), dev(w)
    outs = []
    for _ in range(2):
        dlp = torch.zeros(len(rows), dtype=torch.float32, device="cuda")
        dcl = torch.zeros(len(grp), dtype=torch.float32, device="cuda")
        dcn = torch.zeros(len(grp), dtype=torch.float32, device="cuda")
        B.token_logprobs(B.S1_BF16, dx.data_ptr(), 8, d, dw.data_ptr(), 1e-6, dE.data_ptr(), V, rows, toks, off,
                         grp, dlp.data_ptr(), dcl.data_ptr(), dcn.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        outs.append((dlp.cpu().numpy(), dcn.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


# ----------------------------------------------------------- plan level
def _marker_features(b):
    """One candidate per option: its token read at the question's marker,
    grouped by question."""
    rows, toks, off, grp = [], [], [0], []
    for j in range(b.n_questions):
        r = int(b.cu_seqlens[b.q_seq[j]]) + int(b.q_marker[j])
        for t in b.options_of(j):
            rows.append(r)
            toks.append(int(t))
            off.append(len(rows))
            grp.append(j)
    return rows, toks, off, grp


def _next_token_features(b, rng, n):
    """n targets: a row's next token in its own sequence."""
    rows, toks = [], []
    for _ in range(n):
        i = int(rng.integers(0, b.n_seqs))
        L = int(b.seq_lens[i])
        p = int(rng.integers(0, L - 1))
        r = int(b.cu_seqlens[i]) + p
        rows.append(r)
        toks.append(int(b.token_ids[r + 1]))
    return rows, toks


def _run_plan_features(model, b, rows, toks, off, grp, graph=False, capture=None):
    """Runs (twice when replayed as a graph) with features on; each output
    is (probs, logp, cand logp, cand norm[, final residual rows of capture])."""
    import torch
    plan = model.plan(b)
    Q, nopt = plan.n_questions, plan.n_options
    dp = torch.zeros(max(nopt, 1), dtype=torch.float32, device="cuda")
    dd = torch.zeros((max(Q, 1), 6), dtype=torch.float32, device="cuda")
    dlp = torch.full((len(rows),), float("nan"), dtype=torch.float32, device="cuda")
    dcl = torch.full((max(len(grp), 1),), float("nan"), dtype=torch.float32, device="cuda")
    dcn = torch.full((max(len(grp), 1),), float("nan"), dtype=torch.float32, device="cuda")
    plan.set_features(rows, toks, off, grp, dlp.data_ptr(), dcl.data_ptr(), dcn.data_ptr())
    hid = None
    if capture is not None:
        cfg = model.config
        hid = torch.zeros((cfg.n_layers + 1, len(capture), cfg.d_model), dtype=torch.float32, device="cuda")
        plan.set_capture(np.asarray(capture, np.int32), hid.data_ptr())
    if graph:
        plan.set_graph(True)
    outs = []
    for _ in range(2 if graph else 1):
        plan.run(dp.data_ptr(), dd.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        o = (dp.cpu().numpy()[:nopt].copy(), dlp.cpu().numpy().copy(), dcl.cpu().numpy()[:len(grp)].copy(),
             dcn.cpu().numpy()[:len(grp)].copy())
        if hid is not None:
            o = o + (hid[-1].cpu().numpy().copy(),)
        outs.append(o)
    plan.free()
    return outs


def test_plan_features_tiny_fp32():
    torch = require_gpu()
    shape = shape_of("tiny-fp32")
    w = make_weights(shape)
    b = make_batch("tiny-fp32")
    cfg = s1.make_config(shape, max_tokens=4096)
    model = s1.Model(cfg, w.tensors)
    rng = np.random.default_rng(21)
    rows, toks, off, grp = _marker_features(b)
    nr, nt = _next_token_features(b, rng, 12)
    # multi-token candidates: the next three tokens after a row, two per group
    for g in range(3):
        for _ in range(2):
            r = int(rng.integers(0, b.n_tokens - 4))
            for i in range(3):
                rows.append(r + i)
                toks.append(int(b.token_ids[r + i + 1]))
            off.append(len(rows))
            grp.append(1000 + g)
    rows += nr
    toks += nt
    (probs, lp, cl, cn), = _run_plan_features(model, b, rows, toks, off, grp)
    om = O.OracleModel(shape, w.tensors)
    ids = b.tokens_of(0)
    x, _, _ = om.forward(ids)
    ref_lp, _ = om.token_log_probs(x, rows, toks)
    ref_cl, ref_cn = O.candidate_log_probs(ref_lp, off, grp)
    e = np.abs(lp - ref_lp).max()
    log(f"tiny plan features: max |d logp| {e:.2e}, |d norm| {np.abs(cn - ref_cn).max():.2e}")
    assert e <= 2e-4
    assert np.abs(cl - ref_cl).max() <= 8e-4 and np.abs(cn - ref_cn).max() <= 1.6e-3
    # the option candidates normalised per question are the readout's probabilities
    nopt = int(b.opt_offsets[-1])
    np.testing.assert_allclose(np.exp(cn[:nopt]), probs, atol=2e-5)
    model.free()


def test_plan_features_4b_single_512_graph(gpu_model_4b, oracle_4b_exact):
    """Features at the 4B request, replayed as a HIP graph (twice; both
    replays bit-equal), against the float32 oracle's features of the path's
    own final rows at the kernel tolerance (2e-4 in logp), and the option
    candidates normalised per question equal to the readout's probabilities.
    The final rows themselves are gated layer by layer in test_gpu_3_full."""
    require_gpu()
    b = make_batch("4b-single-512")
    rng = np.random.default_rng(4)
    rows, toks, off, grp = _marker_features(b)
    nr, nt = _next_token_features(b, rng, 29)
    rows += nr
    toks += nt
    u = sorted(set(rows))
    outs = _run_plan_features(gpu_model_4b, b, rows, toks, off, grp, graph=True, capture=u)
    for k in range(4):
        assert np.array_equal(outs[0][k], outs[1][k])
    probs, lp, cl, cn = outs[0][:4]
    final = outs[0][4]
    idx = [u.index(r) for r in rows]
    ref_lp, _ = oracle_4b_exact.token_log_probs(final.astype(np.float64), idx, toks)
    ref_cl, ref_cn = O.candidate_log_probs(ref_lp, off, grp)
    e = np.abs(lp - ref_lp).max()
    log(f"4b plan features on the path's final rows: max |d logp| {e:.2e}, "
        f"|d cand| {np.abs(cl - ref_cl).max():.2e}, |d norm| {np.abs(cn - ref_cn).max():.2e}")
    assert e <= 2e-4
    assert np.abs(cl - ref_cl).max() <= 8e-4 and np.abs(cn - ref_cn).max() <= 1.6e-3
    nopt = int(b.opt_offsets[-1])
    np.testing.assert_allclose(np.exp(cn[:nopt]), probs, atol=2e-5)
