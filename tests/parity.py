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
# bf16 path against an exact float reference: the pages' own allowance for a
# bf16 worker against float32 (Cua-S1 issue, comment on the Rust worker:
# largest difference 0.0065 against an allowance of 0.039)
EXACT_PROB_TOL = 0.039


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


def compare(batch, probs, dec, ref, questions=None, hidden=None, ref_hidden=None, label="",
            ref_exact=None):
    """Returns a dict of the worst metrics; asserts the gates.  ref is the
    oracle in the path's precision (bf16 matrix-product operands for bf16
    models); ref_exact, if given, the oracle without activation rounding,
    checked on probabilities against EXACT_PROB_TOL."""
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
    worst_e, flips_e = 0.0, 0
    if ref_exact is not None:
        for j in qs:
            lo, hi = batch.opt_offsets[j], batch.opt_offsets[j + 1]
            rp = ref_exact["probs"][j]
            worst_e = max(worst_e, float(np.abs(probs[lo:hi] - rp).max()))
            srt = np.sort(rp)
            if srt[-1] - srt[-2] >= MARGIN and int(dec[j]["choice"]) != ref_exact["fields"][j]["choice"]:
                flips_e += 1
    layers = ""
    if hidden is not None:
        layers = " per layer: " + " ".join(f"{rel_l2(hidden[l], ref_hidden[l]):.1e}" for l in range(hidden.shape[0]))
    log(f"{label}: max|dp| {worst_p:.2e}, worst layer rel L2 {worst_h:.2e}, "
        f"argmax checked {checked}, flips {flips}"
        + (f"; vs exact oracle max|dp| {worst_e:.2e}, flips {flips_e}" if ref_exact is not None else "")
        + layers)
    assert worst_p <= PROB_TOL, worst_p
    assert worst_h <= HIDDEN_TOL, worst_h
    assert flips == 0
    assert worst_e <= EXACT_PROB_TOL, worst_e
    return {"max_dp": worst_p, "rel_l2": worst_h, "checked": checked, "max_dp_exact": worst_e}


def oracle_rows(batch, capture):
    """capture: {seq: rows within seq} -> packed row list in capture order."""
    rows = []
    for i, rr in capture.items():
        rows.extend(int(batch.cu_seqlens[i]) + np.asarray(rr, int))
    return rows


def stack_ref_hidden(ref, capture):
    return np.concatenate([ref["hidden"][i] for i in capture], axis=1)


STRICT_LAYERS = 4          # full gates on the first layers (linear and full attention)
DRIFT_FACTOR = 1.5


def compare_full_depth(batch, probs, dec, ref, ref_exact, hidden, ref_hidden, exact_hidden,
                       questions=None, label=""):
    """Gates at full depth.  Two bf16 evaluations of a deep network (this path,
    or the oracle with bf16 operands) each drift from exact arithmetic by the
    bf16 rounding of every layer; their mutual difference grows the same way.
    So: the per-layer 1e-2 gate on the first STRICT_LAYERS layers; at every
    layer, this path's distance from the exact oracle at most DRIFT_FACTOR
    times the bf16 oracle's own distance from it (+2e-3); probabilities within
    an allowance of both oracles -- the pages' bf16-vs-float32 allowance, or
    DRIFT_FACTOR times the bf16 oracle's own probability drift (+5e-3) if that
    is larger; identical choice wherever the exact oracle's margin exceeds
    twice the allowance (an error within it cannot flip such a choice);
    answer fields consistent with this path's probabilities."""
    qs = range(batch.n_questions) if questions is None else list(questions)
    L = hidden.shape[0]
    g_b = [rel_l2(hidden[l], ref_hidden[l]) for l in range(L)]
    g_x = [rel_l2(hidden[l], exact_hidden[l]) for l in range(L)]
    b_x = [rel_l2(ref_hidden[l], exact_hidden[l]) for l in range(L)]
    dp_b = dp_x = dp_bx = 0.0
    for j in qs:
        lo, hi = batch.opt_offsets[j], batch.opt_offsets[j + 1]
        dp_b = max(dp_b, float(np.abs(probs[lo:hi] - ref["probs"][j]).max()))
        dp_x = max(dp_x, float(np.abs(probs[lo:hi] - ref_exact["probs"][j]).max()))
        dp_bx = max(dp_bx, float(np.abs(ref["probs"][j] - ref_exact["probs"][j]).max()))
        f = O.decision_fields(probs[lo:hi].astype(np.float64), int(batch.q_type[j]))
        for key in ("score", "noul", "answer_confidence", "confidence", "entropy_confidence"):
            assert abs(float(dec[j][key]) - f[key]) <= 2e-5 * max(1.0, abs(f[key])), (j, key)
    allow = max(EXACT_PROB_TOL, DRIFT_FACTOR * dp_bx + 5e-3)
    flips_02 = flips_wide = checked = 0
    for j in qs:
        srt = np.sort(ref_exact["probs"][j])
        margin = srt[-1] - srt[-2]
        flip = int(dec[j]["choice"]) != ref_exact["fields"][j]["choice"]
        if margin >= MARGIN:
            checked += 1
            flips_02 += flip
        if margin > 2 * allow:
            flips_wide += flip
    fmt = lambda v: " ".join(f"{x:.1e}" for x in v)
    log(f"{label}: vs bf16 oracle max|dp| {dp_b:.2e}; vs exact oracle max|dp| {dp_x:.2e} "
        f"(bf16 oracle vs exact {dp_bx:.2e}, allowance {allow:.3f}); "
        f"choices with margin >= 0.02: {checked}, flips {flips_02}; flips beyond the allowance band {flips_wide}\n"
        f"  per layer, path vs bf16 oracle:  {fmt(g_b)}\n"
        f"  per layer, path vs exact oracle: {fmt(g_x)}\n"
        f"  per layer, bf16 oracle vs exact: {fmt(b_x)}")
    assert max(g_b[:STRICT_LAYERS + 1]) <= HIDDEN_TOL, g_b[:STRICT_LAYERS + 1]
    for l in range(L):
        assert g_x[l] <= DRIFT_FACTOR * b_x[l] + 2e-3, (l, g_x[l], b_x[l])
    assert dp_x <= allow and dp_b <= allow, (dp_x, dp_b, allow)
    assert flips_wide == 0
    return {"dp_bf16": dp_b, "dp_exact": dp_x, "flips_02": flips_02, "layers_vs_bf16": g_b,
            "layers_vs_exact": g_x}
