"""Row invariance (batch invariance): the arithmetic applied to one row must
not depend on how many other rows share the launch (RFC #114 comment "Plan:
native OmniJev-4B v1.1", design notes: a fixed-GEMM test that rows do not
depend on M, so batched rows keep the order invariance the reference reports
as exactly zero).  Kernel level: every tile configuration of the projection
GEMM gives the same bits for the same rows, whatever M; the two linear-
attention scan schedules give the same bits."""
import numpy as np
import pytest

import oracle as O

from s1_workloads import f32_to_bf16_bits
from tests.gpu_util import dev, dev_bits, host_bits, log, require_gpu, stream_ptr

pytestmark = pytest.mark.gpu

import prefill_only_decision_amd as s1  # noqa: E402
from prefill_only_decision_amd import binding as B  # noqa: E402


def _bits(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("N,K", [(640, 512), (2560, 2048), (1024, 9728)])
def test_gemm_rows_do_not_depend_on_m_or_tile(N, K):
    """Rows 0..M-1 of a GEMM computed at M in {1, 77, 300, 1000} with every
    LDS tile configuration and no K split: all bit-identical."""
    torch = require_gpu()
    rng = np.random.default_rng([N, K])
    Mmax = 1000
    A, W = _bits(rng, (Mmax, K)), _bits(rng, (N, K), 0.05)
    dA, dW = dev_bits(A), dev_bits(W)
    ref = None
    for M in (1000, 300, 77, 1):
        for cfg in range(1, B.gemm_tile_configs()):
            dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            B.gemm_cfg(B.S1_BF16, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K, 1, cfg, stream_ptr())
            torch.cuda.synchronize()
            C = dC.cpu().numpy()
            if ref is None:
                ref = C
            diff = int((C.view(np.uint32) != ref[:M].view(np.uint32)).sum())
            log(f"N={N} K={K} M={M} cfg={cfg}: {diff} elements differ from M=1000 cfg=1")
            assert diff == 0


def test_scan_schedules_agree_to_rounding():
    """The sequential-chunk and the chunk-parallel scan of the same
    sequences agree in their bf16 outputs and to fp32 rounding in their
    final states, but not bit for bit (the chunk-parallel schedule combines
    chunk states in another order): the row-invariant mode therefore runs
    one schedule in every pass."""
    torch = require_gpu()
    rng = np.random.default_rng(77)
    H, dk, lens = 4, 128, [1, 64, 65, 200, 640]
    T = sum(lens)
    qkv = _bits(rng, (T, 3 * H * dk), 1.0)
    lg = np.log(1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    s0 = (rng.standard_normal((len(lens), H, dk, dk)) * 0.1).astype(np.float32)
    d_qkv, d_lg, d_s0 = dev_bits(qkv), dev(lg), dev(s0)
    base = d_qkv.data_ptr()
    outs = []
    for chunked in (False, True):
        d_o = torch.zeros((T, H * dk), dtype=torch.int16, device="cuda")
        d_sf = torch.zeros((len(lens), H, dk, dk), dtype=torch.float32, device="cuda")
        if chunked:
            B.la_scan_chunked(base, base + 2 * H * dk, base + 4 * H * dk, 3 * H * dk, d_lg.data_ptr(),
                              d_o.data_ptr(), T, H, cu, d_s0.data_ptr(), d_sf.data_ptr(), stream_ptr())
        else:
            B.la_scan(B.S1_BF16, base, base + 2 * H * dk, base + 4 * H * dk, 3 * H * dk, d_lg.data_ptr(),
                      d_o.data_ptr(), T, H, dk, dk, cu, d_s0.data_ptr(), d_sf.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        outs.append((host_bits(d_o), d_sf.cpu().numpy()))
    do = int((outs[0][0] != outs[1][0]).sum())
    ds = int((outs[0][1].view(np.uint32) != outs[1][1].view(np.uint32)).sum())
    rel = np.linalg.norm(outs[0][1] - outs[1][1]) / np.linalg.norm(outs[1][1])
    log(f"scan schedules: {do} output elements and {ds} state elements differ (state rel L2 {rel:.1e})")
    assert do <= T * H * dk // 1000 and rel < 1e-6


# ------------------------------------------------------------ plan level
def _run(model, batch, rows, invariant=True):
    """Whole request through a plan; returns probs, decision bytes and the
    residual stream of `rows` (packed indices) after every layer."""
    import torch
    plan = model.plan(batch)
    plan.set_invariant(invariant)
    nopt, Q = plan.n_options, plan.n_questions
    dp = torch.zeros(max(nopt, 1), dtype=torch.float32, device="cuda")
    dd = torch.zeros((max(Q, 1), 6), dtype=torch.float32, device="cuda")
    L, d = model.config.n_layers, model.config.d_model
    hid = torch.zeros((L + 1, len(rows), d), dtype=torch.float32, device="cuda")
    plan.set_capture(np.asarray(rows, np.int32), hid.data_ptr())
    plan.run(dp.data_ptr(), dd.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    out = dp.cpu().numpy()[:nopt].copy(), dd.cpu().numpy()[:Q].copy(), hid.cpu().numpy()
    plan.free()
    return out


def _same_bits(a, b):
    return int((np.ascontiguousarray(a).view(np.uint32) != np.ascontiguousarray(b).view(np.uint32)).sum())


def _alone(b, i):
    """Sequence i of a packed batch as a request of its own."""
    from s1_workloads.batch import _assemble
    qs = [(0, int(b.q_marker[j]), int(b.q_type[j]), b.options_of(j)) for j in range(b.n_questions)
          if int(b.q_seq[j]) == i]
    return _assemble([b.tokens_of(i)], [-1], qs)


def _question_slices(b, i):
    return [(int(b.opt_offsets[j]), int(b.opt_offsets[j + 1])) for j in range(b.n_questions) if int(b.q_seq[j]) == i]


def test_packed_sequences_equal_each_alone_bitwise(gpu_model_4b):
    """Row-invariant mode: a sequence packed with 15 others gives bitwise the
    outputs it gives alone, at every layer."""
    require_gpu()
    from s1_workloads import make_batch
    b = make_batch("4b-varlen-16")
    sample = [9, 4, 15]
    rng = np.random.default_rng(8)
    rows_in = {i: np.unique(np.concatenate([rng.choice(int(b.seq_lens[i]), 6, replace=False), [0, int(b.seq_lens[i]) - 1]]))
               for i in sample}
    packed_rows = np.concatenate([int(b.cu_seqlens[i]) + rows_in[i] for i in sample])
    probs, dec, hid = _run(gpu_model_4b, b, packed_rows)
    k = 0
    for i in sample:
        p1, d1, h1 = _run(gpu_model_4b, _alone(b, i), rows_in[i])
        n = len(rows_in[i])
        dh = _same_bits(hid[:, k:k + n], h1)
        sl = _question_slices(b, i)
        dp = sum(_same_bits(probs[lo:hi], p1[a:c]) for (lo, hi), (a, c) in
                 zip(sl, [(s - sl[0][0], e - sl[0][0]) for s, e in sl]))
        log(f"sequence {i} ({int(b.seq_lens[i])} tokens): {dh} hidden and {dp} probability values differ")
        assert dh == 0 and dp == 0
        k += n


def test_branches_equal_plain_forward_bitwise(gpu_model_4b):
    """Row-invariant mode: a branch continued from the shared prefix gives
    bitwise the outputs of the plain forward of prefix + branch."""
    require_gpu()
    from s1_workloads import make_batch
    from s1_workloads.batch import _assemble
    b = make_batch("4b-branch-4096x20")
    P = int(b.seq_lens[0])
    branch_rows = np.array([0, 31, 63])
    sample = [1, 20]
    packed_rows = np.concatenate([int(b.cu_seqlens[i]) + branch_rows for i in sample])
    probs, dec, hid = _run(gpu_model_4b, b, packed_rows)
    for k, i in enumerate(sample):
        qs = [(0, P + int(b.q_marker[j]), int(b.q_type[j]), b.options_of(j)) for j in range(b.n_questions)
              if int(b.q_seq[j]) == i]
        plain = _assemble([np.concatenate([b.tokens_of(0), b.tokens_of(i)])], [-1], qs)
        p1, d1, h1 = _run(gpu_model_4b, plain, P + branch_rows)
        dh = _same_bits(hid[:, 3 * k:3 * k + 3], h1)
        sl = _question_slices(b, i)
        dp = sum(_same_bits(probs[lo:hi], p1[lo - sl[0][0]:hi - sl[0][0]]) for lo, hi in sl)
        log(f"branch {i}: {dh} hidden and {dp} probability values differ from the plain forward")
        assert dh == 0 and dp == 0


def test_invariant_mode_against_oracle(gpu_model_4b, oracle_4b_exact):
    """The row-invariant schedule under the fixed gates against the float32
    oracle: every layer from the oracle's input within 1e-2, its readout
    within 1e-2 with no choice flip where the margin >= 0.02; end-to-end
    answers printed."""
    require_gpu()
    from s1_workloads import make_batch, shape_of
    from tests.parity import decision_gate, layer_local_gate, run_gpu
    shape = shape_of("4b-single-512")
    b = make_batch("4b-single-512")
    cap = {0: np.arange(512)}
    ref = O.prefill_decide(oracle_4b_exact, b, capture=cap)
    probs, dec, _ = run_gpu(gpu_model_4b, b, invariant=True)
    decision_gate(b, probs, dec, ref, None, label="4b-single-512 row-invariant end to end")
    layer_local_gate(gpu_model_4b, b, ref, [0], cap, shape.n_layers, shape.d_model,
                     label="4b-single-512 row-invariant", invariant=True)
