"""Run a request through the C ABI (resident-input plan) and compare it with
the oracle under the gates: per-layer hidden-state relative L2 <= 1e-2,
option probabilities max-abs <= 1e-2, identical choice wherever the oracle's
top-2 margin is >= 0.02 (RFC #114, section 6: proposed numerical gates)."""
import numpy as np

import oracle as O
from tests.gpu_util import log, rel_l2, stream_ptr

HIDDEN_TOL = 1e-2
PROB_TOL = 1e-2
MARGIN = 0.02


def run_gpu(model, batch, capture_rows=None, n_layers=None, d=None):
    import torch
    import prefill_only_decision_amd as s1
    plan = model.plan(batch)
    Q, nopt = plan.n_questions, plan.n_options
    dp = torch.zeros(max(nopt, 1), dtype=torch.float32, device="cuda")
    dd = torch.zeros((max(Q, 1), 6), dtype=torch.float32, device="cuda")
    hid = None
    if capture_rows is not None and len(capture_rows):
        hid = torch.zeros((n_layers + 1, len(capture_rows), d), dtype=torch.float32, device="cuda")
        plan.set_capture(np.asarray(capture_rows, np.int32), hid.data_ptr())
    plan.run(dp.data_ptr(), dd.data_ptr(), stream_ptr())
    torch.cuda.synchronize()
    probs = dp.cpu().numpy()[:nopt]
    dec = dd.cpu().numpy()[:Q].copy().view(np.uint8).view(s1.DECISION_DTYPE).reshape(Q)
    plan.free()
    return probs, dec, (hid.cpu().numpy() if hid is not None else None)


def compare(batch, probs, dec, ref, questions=None, hidden=None, ref_hidden=None, label=""):
    """Returns a dict of the worst metrics; asserts the gates."""
    qs = range(batch.n_questions) if questions is None else questions
    worst_p, flips, checked = 0.0, 0, 0
    for j in qs:
        lo, hi = batch.opt_offsets[j], batch.opt_offsets[j + 1]
        rp = ref["probs"][j]
        worst_p = max(worst_p, float(np.abs(probs[lo:hi] - rp).max()))
        srt = np.sort(rp)
        if srt[-1] - srt[-2] >= MARGIN:
            checked += 1
            if int(dec[j]["choice"]) != ref["fields"][j]["choice"]:
                flips += 1
        # the answer fields must be those of the GPU's own probabilities
        f = O.decision_fields(probs[lo:hi].astype(np.float64), int(batch.q_type[j]))
        for key in ("score", "noul", "answer_confidence", "confidence", "entropy_confidence"):
            assert abs(float(dec[j][key]) - f[key]) <= 2e-5 * max(1.0, abs(f[key])), (j, key)
    worst_h = 0.0
    if hidden is not None:
        for l in range(hidden.shape[0]):
            worst_h = max(worst_h, rel_l2(hidden[l], ref_hidden[l]))
    log(f"{label}: max|dp| {worst_p:.2e}, worst layer rel L2 {worst_h:.2e}, "
        f"argmax checked {checked}, flips {flips}")
    assert worst_p <= PROB_TOL, worst_p
    assert worst_h <= HIDDEN_TOL, worst_h
    assert flips == 0
    return {"max_dp": worst_p, "rel_l2": worst_h, "checked": checked}


def oracle_rows(batch, capture):
    """capture: {seq: rows within seq} -> packed row list in capture order."""
    rows = []
    for i, rr in capture.items():
        rows.extend(int(batch.cu_seqlens[i]) + np.asarray(rr, int))
    return rows


def stack_ref_hidden(ref, capture):
    return np.concatenate([ref["hidden"][i] for i in capture], axis=1)
