"""Pins of the CPU oracle against facts it does not compute itself: closed
forms, brute-force loops on tiny inputs, library routines, and the values the
sys1rust README prints for the readout's special cases.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                lhs, rhs = line.split("|")
                yield lhs.split(), rhs.split()


# --------------------------------------------------------------------- bf16
def test_bf16_rounding_golden():
    for lhs, rhs in _golden_rows("bf16_rounding.txt"):
        x = eval(" ".join(lhs), {"__builtins__": {}})
        assert O.round_to_bf16_bits(np.array([x]))[0] == int(rhs[0], 16), lhs


def test_bf16_rounding_matches_torch_for_float32_inputs():
    # For inputs that are already float32, one-step rounding from float64 and
    # torch's float32 -> bfloat16 conversion (RNE) must agree bit for bit.
    x = (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-6, 4, 200_000)).astype(np.float32)
    ours = O.round_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000], np.uint16)
    assert O.bf16_bits_to_float(bits).tolist() == [1.0, -2.0, 0.25, 0.0, -0.0]


# ------------------------------------------------------------------ rmsnorm
def test_rmsnorm_constant_vector_closed_form():
    c, eps = 0.37, 1e-6
    x = np.full((1, 64), c)
    w = rng.standard_normal(64)
    np.testing.assert_allclose(O.rms_norm(x, w, eps)[0], w * c / math.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm_matches_torch():
    x = rng.standard_normal((7, 256))
    w = rng.standard_normal(256)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (256,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-6), ref.numpy(), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------- rope
def test_rope_equals_complex_rotation():
    T, H, hd, base = 9, 3, 16, 10000.0
    a = rng.standard_normal((T, H, hd))
    pos = rng.integers(0, 5000, T)
    half = hd // 2
    z = a[..., :half] + 1j * a[..., half:]
    theta = np.array([base ** (-(2 * i) / hd) for i in range(half)])
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    np.testing.assert_allclose(O.rope_rotate_half(a, pos, base), ref, rtol=1e-10, atol=1e-12)


def test_rope_position_zero_identity_and_hand_value():
    a = rng.standard_normal((1, 2, 8))
    np.testing.assert_array_equal(O.rope_rotate_half(a, np.array([0]), 10000.0), a)
    a = np.array([[[1.0, 0.0]]])      # hd = 2: theta_0 = 1, pos 1 -> angle 1 rad
    out = O.rope_rotate_half(a, np.array([1]), 10000.0)[0, 0]
    np.testing.assert_allclose(out, [math.cos(1.0), math.sin(1.0)], rtol=1e-15)


def test_rope_scores_depend_on_relative_position_only():
    hd = 32
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    def score(pq, pk):
        return float((O.rope_rotate_half(q, np.array([pq]), 10000.0) *
                      O.rope_rotate_half(k, np.array([pk]), 10000.0)).sum())
    assert abs(score(10, 3) - score(4107, 4100)) < 1e-9
    assert abs(score(10, 3) - score(11, 3)) > 1e-6


# --------------------------------------------------------------------- scan
def _qkvg(T, H=2, dk=4, dv=3, gate=None):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(0.02, 0.98, (T, H)) if gate is None else np.full((T, H), gate)
    return q, k, v, g


def test_scan_scalar_golden():
    rows = list(_golden_rows("scan_scalar_example.txt"))
    q, k, v, g = (np.array([float(r[0][i]) for r in rows]) for i in range(4))
    o_exp = [float(r[1][0]) for r in rows]
    S_exp = float(rows[-1][1][1])
    sh = lambda a: a.reshape(-1, 1, 1)
    for fn in (O.la_scan_recurrent, O.la_scan_unrolled):
        o, S = fn(sh(q), sh(k), sh(v), g.reshape(-1, 1))
        np.testing.assert_allclose(o[:, 0, 0], o_exp, rtol=1e-14)
        assert abs(S[0, 0, 0] - S_exp) < 1e-14


@pytest.mark.parametrize("fn", [O.la_scan_recurrent, O.la_scan_unrolled])
def test_scan_gate_one_is_causal_linear_attention(fn):
    q, k, v, g = _qkvg(11, gate=1.0)
    o, _ = fn(q, k, v, g)
    for t in range(11):
        for h in range(2):
            ref = sum(float(np.dot(q[t, h], k[s, h])) * v[s, h] for s in range(t + 1))
            np.testing.assert_allclose(o[t, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fn", [O.la_scan_recurrent, O.la_scan_unrolled])
def test_scan_gate_zero_keeps_only_current_token(fn):
    q, k, v, g = _qkvg(9, gate=0.0)
    S0 = rng.standard_normal((2, 4, 3))
    o, S = fn(q, k, v, g, S0)
    ref = np.einsum("thk,thk->th", q, k)[:, :, None] * v
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, k[-1][:, :, None] * v[-1][:, None, :], rtol=1e-12)


def test_scan_pure_decay_of_initial_state():
    T = 7
    q, k, v, g = _qkvg(T)
    k[:] = 0.0
    S0 = rng.standard_normal((2, 4, 3))
    for fn in (O.la_scan_recurrent, O.la_scan_unrolled):
        o, S = fn(q, k, v, g, S0)
        decay = np.cumprod(g, axis=0)             # prod_{r<=t} g_r
        ref = decay[:, :, None] * np.einsum("hkv,thk->thv", S0, q)
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S, decay[-1][:, None, None] * S0, rtol=1e-12)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 300])
def test_scan_unrolled_equals_recurrence(T):
    q, k, v, g = _qkvg(T, H=3, dk=8, dv=5)
    S0 = rng.standard_normal((3, 8, 5))
    for init in (None, S0):
        o1, S1 = O.la_scan_recurrent(q, k, v, g, init)
        o2, S2 = O.la_scan_unrolled(q, k, v, g, init)
        np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(S2, S1, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("P", [0, 1, 37, 64, 100])
def test_scan_continuation(P):
    q, k, v, g = _qkvg(100, H=2, dk=6, dv=4)
    o_full, S_full = O.la_scan_recurrent(q, k, v, g)
    oa, Sa = O.la_scan_unrolled(q[:P], k[:P], v[:P], g[:P])
    ob, Sb = O.la_scan_unrolled(q[P:], k[P:], v[P:], g[P:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o_full, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(Sb, S_full, rtol=1e-10, atol=1e-10)


def test_scan_segmented_equals_recurrence():
    q, k, v, g = _qkvg(1100, H=2, dk=5, dv=3)
    S0 = rng.standard_normal((2, 5, 3))
    o1, S1 = O.la_scan_recurrent(q, k, v, g, S0)
    for seg in (1, 64, 512, 2000):
        o2, S2 = O.la_scan_segmented(q, k, v, g, S0, segment=seg)
        np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(S2, S1, rtol=1e-10, atol=1e-10)


def test_scan_strong_decay_no_overflow():
    # gates ~0.02 over 2000 tokens: products underflow; differences must not
    q, k, v, _ = _qkvg(2000, H=1, dk=4, dv=4)
    g = np.full((2000, 1), 0.02)
    o, S = O.la_scan_unrolled(q, k, v, g)
    o2, S2 = O.la_scan_recurrent(q, k, v, g)
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o, o2, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- attention
def _attn_loops(q, k, v, qp, kp):
    Tq, Hq, hd = q.shape
    grp = Hq // k.shape[1]
    out = np.zeros_like(q)
    for t in range(Tq):
        for h in range(Hq):
            kv = h // grp
            sc = [sum(q[t, h, d] * k[s, kv, d] for d in range(hd)) / math.sqrt(hd)
                  if kp[s] <= qp[t] else None for s in range(k.shape[0])]
            m = max(x for x in sc if x is not None)
            w = [math.exp(x - m) if x is not None else 0.0 for x in sc]
            Z = sum(w)
            for d in range(hd):
                out[t, h, d] = sum(w[s] * v[s, kv, d] for s in range(k.shape[0])) / Z
    return out


def test_attention_brute_force_loops_gqa():
    q = rng.standard_normal((5, 4, 4))
    k = rng.standard_normal((5, 2, 4))
    v = rng.standard_normal((5, 2, 4))
    pos = np.arange(5)
    np.testing.assert_allclose(O.causal_attention(q, k, v, pos, pos),
                               _attn_loops(q, k, v, pos, pos), rtol=1e-12)


def test_attention_matches_torch_sdpa():
    T, H, hd = 37, 4, 16
    q, k, v = (rng.standard_normal((T, H, hd)) for _ in range(3))
    pos = np.arange(T)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a).permute(1, 0, 2) for a in (q, k, v)), is_causal=True)
    np.testing.assert_allclose(O.causal_attention(q, k, v, pos, pos),
                               ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_attention_special_cases():
    v = rng.standard_normal((1, 2, 8))
    q = rng.standard_normal((1, 2, 8))
    k = rng.standard_normal((1, 2, 8))
    np.testing.assert_allclose(O.causal_attention(q, k, v, [0], [0]), v, rtol=1e-15)
    # identical keys: uniform weights over the visible prefix
    T = 6
    q = rng.standard_normal((T, 2, 8))
    k = np.repeat(rng.standard_normal((1, 2, 8)), T, axis=0)
    v = rng.standard_normal((T, 2, 8))
    o = O.causal_attention(q, k, v, np.arange(T), np.arange(T))
    ref = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None, None]
    np.testing.assert_allclose(o, ref, rtol=1e-12)


def test_attention_gqa_equals_mha_with_repeated_kv():
    q = rng.standard_normal((12, 8, 16))
    k = rng.standard_normal((12, 2, 16))
    v = rng.standard_normal((12, 2, 16))
    pos = np.arange(12)
    ref = O.causal_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), pos, pos)
    np.testing.assert_allclose(O.causal_attention(q, k, v, pos, pos), ref, rtol=1e-14)


def test_attention_prefix_keys_equal_full_rows():
    T, P = 30, 17
    q, k, v = (rng.standard_normal((T, 2, 8)) for _ in range(3))
    pos = np.arange(T)
    full = O.causal_attention(q, k, v, pos, pos)
    part = O.causal_attention(q[P:], k, v, pos[P:], pos)
    np.testing.assert_allclose(part, full[P:], rtol=1e-13)


# --------------------------------------------------------------------- lora
def test_lora_merge_associativity_and_zero_b():
    W = rng.standard_normal((24, 40))
    A = rng.standard_normal((8, 40))
    B = rng.standard_normal((24, 8))
    x = rng.standard_normal((5, 40))
    Wm = O.lora_merge(W, A, B, 16.0, 8)
    np.testing.assert_allclose(x @ Wm.T, x @ W.T + 2.0 * ((x @ A.T) @ B.T), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(O.lora_merge(W, A, np.zeros_like(B), 16.0, 8), W)


def test_bf16_merge_is_within_half_ulp():
    W = O.bf16_bits_to_float(rng.integers(0x3000, 0x3D00, (64, 80)).astype(np.uint16))
    A = rng.standard_normal((32, 80)) * 0.02
    B = rng.standard_normal((64, 32)) * 0.02
    exact = O.lora_merge(W, A, B, 64.0, 32)
    r = O.bf16_bits_to_float(O.round_to_bf16_bits(exact))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
    assert (np.abs(r - exact) <= 0.5 * ulp * (1 + 1e-12)).all()


# ------------------------------------------------------------------- swiglu
def test_silu_hand_values():
    u = np.array([[1.0]])
    one = np.array([[1.0]])
    assert abs(O.swiglu(u, one, one, one)[0, 0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert O.swiglu(np.array([[0.0]]), one, one, one)[0, 0] == 0.0
    x = rng.standard_normal((3, 10))
    wg, wu, wd = rng.standard_normal((6, 10)), rng.standard_normal((6, 10)), rng.standard_normal((10, 6))
    a = torch.from_numpy(x @ wg.T)
    ref = (torch.nn.functional.silu(a).numpy() * (x @ wu.T)) @ wd.T
    np.testing.assert_allclose(O.swiglu(x, wg, wu, wd), ref, rtol=1e-12)


# ------------------------------------------------------------------ readout
def test_readout_golden_special_cases():
    for lhs, rhs in _golden_rows("readout_special_cases.txt"):
        qtype, K = int(lhs[0]), int(lhs[1])
        z = np.array([float(t) for t in lhs[2].split(",")])
        f = O.decision_fields(O.softmax(z), qtype)
        assert abs(f["confidence"] - float(rhs[0])) < 1e-12, lhs
        assert abs(f["answer_confidence"] - float(rhs[1])) < 1e-12, lhs


def test_readout_invariants():
    for K in (2, 3, 7, 26):
        z = rng.standard_normal(K) * 3
        p = O.softmax(z)
        assert abs(p.sum() - 1.0) < 1e-12
        f = O.decision_fields(p, O.QTYPE_SCORE)
        assert f["choice"] == int(np.argmax(z))
        assert 0.0 <= f["score"] <= K - 1
        assert 0.0 <= f["entropy_confidence"] <= 1.0
        perm = rng.permutation(K)
        np.testing.assert_allclose(O.softmax(z[perm]), p[perm], rtol=1e-12)
    # K = 2: P(yes) is the logistic of the logit difference
    z = np.array([0.7, -1.9])
    assert abs(O.decision_fields(O.softmax(z), O.QTYPE_NOUL)["noul"] - 1 / (1 + math.exp(-2.6))) < 1e-14
    # one-hot at level 3 of 5: expected level is exactly 3
    assert abs(O.decision_fields(O.softmax(np.array([0, 0, 0, 300.0, 0])), O.QTYPE_SCORE)["score"] - 3) < 1e-12
    # exact tie: lowest index wins
    assert O.decision_fields(O.softmax(np.array([1.0, 2.0, 2.0])), O.QTYPE_CHOICE)["choice"] == 1


def test_readout_applies_final_norm_and_tied_rows():
    d = 16
    h = rng.standard_normal(d)
    w = rng.standard_normal(d)
    E = rng.standard_normal((3, d))
    p, f = O.readout(h, w, E, 1e-6, O.QTYPE_CHOICE)
    hn = h / math.sqrt(float(np.mean(h * h)) + 1e-6) * w
    z = [float(np.dot(E[i], hn)) for i in range(3)]
    Z = sum(math.exp(t) for t in z)
    np.testing.assert_allclose(p, [math.exp(t) / Z for t in z], rtol=1e-12)


# ---------------------------------------------- full-vocabulary log-probs
def _loop_log_probs(h, w, E, eps, rows, tokens):
    """Brute force with scalar loops: final norm, every logit, log-sum-exp."""
    out = []
    for r, t in zip(rows, tokens):
        x = h[r]
        ms = sum(float(v) * float(v) for v in x) / len(x)
        hn = [float(x[i]) / math.sqrt(ms + eps) * float(w[i]) for i in range(len(x))]
        z = [sum(float(E[v][i]) * hn[i] for i in range(len(x))) for v in range(len(E))]
        out.append(z[t] - math.log(sum(math.exp(zv) for zv in z)))
    return out


def test_vocab_log_probs_brute_force_loops():
    R, V, d = 3, 37, 8
    h = rng.standard_normal((R, d)) * 2
    w = rng.standard_normal(d)
    E = rng.standard_normal((V, d))
    rows = [0, 2, 1, 2, 0]
    toks = [5, 36, 0, 17, 5]
    logp, lse = O.vocab_log_probs(h, w, E, 1e-6, rows, toks, chunk=10)
    np.testing.assert_allclose(logp, _loop_log_probs(h, w, E, 1e-6, rows, toks), rtol=1e-12)
    assert lse.shape == (R,)


def test_vocab_log_probs_normalise_over_the_whole_vocabulary():
    R, V, d = 4, 50, 16
    h = rng.standard_normal((R, d))
    w = rng.uniform(0.5, 1.5, d)
    E = rng.standard_normal((V, d)) * 3
    rows = np.repeat(np.arange(R), V)
    toks = np.tile(np.arange(V), R)
    logp, _ = O.vocab_log_probs(h, w, E, 1e-6, rows, toks, chunk=7)
    np.testing.assert_allclose(np.exp(logp).reshape(R, V).sum(axis=1), 1.0, rtol=1e-12)
    assert (logp < 0).all()


def test_vocab_log_probs_library_log_softmax_identity_head():
    # E = s * I (V = d), unit gains and rows of mean square 1: the logits are
    # s * h / sqrt(1 + eps), so the features are scipy's log_softmax of them,
    # also at logits far beyond float64's exp range.
    from scipy.special import log_softmax
    d, eps = 24, 1e-6
    for s in (1.0, 40.0, 2000.0):
        h = rng.standard_normal((2, d))
        h /= np.sqrt(np.mean(h * h, axis=1, keepdims=True))
        rows = np.repeat([0, 1], d)
        toks = np.tile(np.arange(d), 2)
        logp, lse = O.vocab_log_probs(h, np.ones(d), s * np.eye(d), eps, rows, toks, chunk=5)
        ref = log_softmax(s * h / math.sqrt(1 + eps), axis=1).reshape(-1)
        assert np.isfinite(logp).all() and np.isfinite(lse).all()
        np.testing.assert_allclose(logp, ref, rtol=1e-12, atol=1e-12 * s)


def test_vocab_log_probs_identical_rows_give_minus_log_v():
    V, d = 1000, 12
    E = np.tile(rng.standard_normal(d), (V, 1))
    h = rng.standard_normal((2, d)) * 5
    logp, _ = O.vocab_log_probs(h, rng.standard_normal(d), E, 1e-6, [0, 1, 1], [0, 999, 512])
    np.testing.assert_allclose(logp, -math.log(V), rtol=1e-13)


def test_vocab_log_probs_bf16_embedding_and_chunking():
    # bf16 bit patterns decode per chunk; every chunk size (including one that
    # leaves a ragged last chunk) gives the same numbers as the decoded matrix.
    V, d = 301, 32
    Ef = rng.standard_normal((V, d)) * 0.5
    bits = O.round_to_bf16_bits(Ef)
    h = rng.standard_normal((3, d))
    w = rng.standard_normal(d)
    rows, toks = [0, 1, 2, 2], [300, 0, 150, 7]
    ref, ref_lse = O.vocab_log_probs(h, w, O.bf16_bits_to_float(bits), 1e-6, rows, toks, chunk=V)
    for chunk in (1, 64, 100, 301, 4096):
        got, lse = O.vocab_log_probs(h, w, bits, 1e-6, rows, toks, chunk=chunk)
        np.testing.assert_allclose(got, ref, rtol=1e-13)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_vocab_log_probs_option_softmax_equals_readout():
    # Normalising the options' full-vocabulary log-probabilities across the
    # options gives back the readout's option softmax: the vocabulary
    # denominator cancels.
    V, d = 200, 16
    E = rng.standard_normal((V, d))
    h = rng.standard_normal(d)
    w = rng.standard_normal(d)
    opts = [17, 3, 150, 88]
    p, _ = O.readout(h, w, E[opts], 1e-6, O.QTYPE_CHOICE)
    logp, _ = O.vocab_log_probs(h[None], w, E, 1e-6, [0] * 4, opts)
    _, norm = O.candidate_log_probs(logp, [0, 1, 2, 3, 4], [0, 0, 0, 0])
    np.testing.assert_allclose(np.exp(norm), p, rtol=1e-12)
    assert (logp < np.log(p)).all()     # the vocabulary holds other tokens too


def test_candidate_log_probs_hand_values():
    logp = np.log([0.5, 0.25, 0.1, 0.2, 0.4])
    # group 7: candidate 0 = tokens 0, 1 (prob 0.125), candidate 2 = token 4 (0.4)
    # group 3: candidate 1 = tokens 2, 3 (0.02), candidate 3 = nothing (score 0)
    lp, norm = O.candidate_log_probs(logp, [0, 2, 4, 5, 5], [7, 3, 7, 3])
    np.testing.assert_allclose(lp, np.log([0.125, 0.02, 0.4, 1.0]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(np.exp(norm), [0.125 / 0.525, 0.02 / 1.02, 0.4 / 0.525, 1 / 1.02],
                               rtol=1e-13)
    # a question with one candidate normalises to log 1 = 0
    _, n1 = O.candidate_log_probs([-3.0, -4.0], [0, 2], [5])
    assert n1[0] == 0.0


# ------------------------------------------------------- Gated DeltaNet
def _gdn_inputs(T, H=2, dk=8, dv=6, seed=0):
    r = np.random.default_rng(seed)
    q = O.l2_normalize(r.standard_normal((T, H, dk)))
    k = O.l2_normalize(r.standard_normal((T, H, dk)))
    v = r.standard_normal((T, H, dv))
    g = r.uniform(0.6, 1.0, (T, H))
    beta = r.uniform(0.05, 0.95, (T, H))
    S0 = r.standard_normal((H, dk, dv)) * 0.3
    return q, k, v, g, beta, S0


@pytest.mark.parametrize("T,chunk", [(1, 64), (7, 3), (64, 64), (150, 64), (37, 1)])
def test_gdn_chunked_equals_recurrence(T, chunk):
    q, k, v, g, beta, S0 = _gdn_inputs(T, seed=T)
    o1, s1 = O.gdn_recurrent(q, k, v, g, beta, S0)
    o2, s2 = O.gdn_chunked(q, k, v, g, beta, S0, chunk=chunk)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s2, s1, rtol=1e-10, atol=1e-12)


def test_gdn_without_writes_is_pure_decay():
    q, k, v, g, beta, S0 = _gdn_inputs(20)
    o, S = O.gdn_recurrent(q, k, v, g, np.zeros_like(beta), S0)
    gam = np.cumprod(g, axis=0)
    np.testing.assert_allclose(S, gam[-1][:, None, None] * S0, rtol=1e-12)
    np.testing.assert_allclose(o, gam[:, :, None] * np.einsum("hkv,thk->thv", S0, q), rtol=1e-12, atol=1e-14)


def test_gdn_orthonormal_keys_are_stored_exactly():
    # g = 1, beta = 1: writing v_i under orthonormal keys k_i stores each
    # exactly (a delta rule write replaces the value read under its key)
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :n].T[:, None, :]                      # [n, 1, dk]
    v = rng.standard_normal((n, 1, dv))
    one = np.ones((n, 1))
    o, S = O.gdn_recurrent(k, k, v, one, one)       # query = the key just written
    np.testing.assert_allclose(o, v, atol=1e-12)
    np.testing.assert_allclose(np.einsum("kv,nk->nv", S[0], k[:, 0]), v[:, 0], atol=1e-12)


def test_gdn_rewrite_under_one_key():
    # same unit key twice: beta = 1 replaces the first value; beta = 1/2
    # moves the stored value half way each time (closed forms)
    dk = 4
    kk = O.l2_normalize(rng.standard_normal(dk), eps=0.0)
    k = np.tile(kk, (2, 1, 1))
    v = rng.standard_normal((2, 1, 3))
    _, S = O.gdn_recurrent(k, k, v, np.ones((2, 1)), np.ones((2, 1)))
    np.testing.assert_allclose(S[0].T @ kk, v[1, 0], atol=1e-12)
    vv = np.tile(v[:1], (2, 1, 1))
    _, S = O.gdn_recurrent(k, k, vv, np.ones((2, 1)), np.full((2, 1), 0.5))
    np.testing.assert_allclose(S[0].T @ kk, 0.75 * v[0, 0], atol=1e-12)


def test_gdn_continuation():
    q, k, v, g, beta, S0 = _gdn_inputs(90, seed=5)
    o, S = O.gdn_recurrent(q, k, v, g, beta, S0)
    oa, Sa = O.gdn_chunked(q[:41], k[:41], v[:41], g[:41], beta[:41], S0)
    ob, Sb = O.gdn_chunked(q[41:], k[41:], v[41:], g[41:], beta[41:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Sb, S, rtol=1e-10, atol=1e-12)


def test_causal_conv_matches_torch_and_continues():
    T, C, W = 23, 10, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    y, hist = O.causal_conv_silu(x, w)
    xt = torch.from_numpy(x.T[None])                                 # [1, C, T]
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (W - 1, 0)),
                                     torch.from_numpy(w[:, None, :]), groups=C)
    np.testing.assert_allclose(y, torch.nn.functional.silu(ref)[0].numpy().T, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hist, x[-(W - 1):])
    ya, ha = O.causal_conv_silu(x[:9], w)
    yb, hb = O.causal_conv_silu(x[9:], w, ha)
    np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-12)
    # the current-token tap alone is a plain SiLU
    e = np.zeros((C, W))
    e[:, W - 1] = 1.0
    np.testing.assert_allclose(O.causal_conv_silu(x, e)[0], x / (1 + np.exp(-x)), rtol=1e-12)


def test_l2_normalize():
    x = rng.standard_normal((5, 3, 16)) * 7
    y = O.l2_normalize(x, eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-12)
