"""Whole-model checks of the CPU oracle on the tiny fp32 shape (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from s1_workloads import make_weights, make_batch, shape_of
from s1_workloads.batch import random_batch


@pytest.fixture(scope="module")
def tiny():
    shape = shape_of("tiny-fp32")
    return shape, make_weights(shape)


def test_generator_is_thread_count_independent(tiny):
    shape, w = tiny
    w1 = make_weights(shape, threads=1)
    for n in w.tensors:
        assert np.array_equal(w.tensors[n], w1.tensors[n]), n


def test_workload_batches_are_valid():
    for name in ("tiny-fp32", "4b-single-512", "4b-varlen-16", "4b-branch-4096x20",
                 "27b-single-1024"):
        b = make_batch(name)
        V = shape_of(name).vocab
        lens = b.seq_lens
        assert (b.token_ids >= 0).all() and (b.token_ids < V).all()
        for j in range(b.n_questions):
            i = b.q_seq[j]
            assert 0 <= b.q_marker[j] < lens[i]
            opts = b.options_of(j)
            assert len(set(opts.tolist())) == len(opts) >= 2
            if b.q_type[j] == O.QTYPE_NOUL:
                assert len(opts) == 2
    b = make_batch("4b-branch-4096x20")
    assert b.n_tokens == 4096 + 20 * 64 and (b.prefix_of[1:] == 0).all()
    b = make_batch("4b-varlen-16")
    assert b.n_seqs == 16 and (b.seq_lens >= 256).all() and (b.seq_lens <= 2048).all()


def _torch_forward(shape, tensors, ids):
    """An independent formulation of the tiny hybrid in PyTorch CPU ops
    (F.linear, F.rms_norm, F.scaled_dot_product_attention, a step loop for
    the recurrence, complex-number RoPE), float64, with LoRA applied unmerged."""
    F = torch.nn.functional
    t = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in tensors.items()}
    s = shape
    sc = s.lora_alpha / s.lora_rank

    def lin(name, x):
        y = F.linear(x, t[name])
        if name + ".lora_A" in t:
            y = y + sc * F.linear(F.linear(x, t[name + ".lora_A"]), t[name + ".lora_B"])
        return y

    def rope(a, pos):
        hd = a.shape[-1]
        half = hd // 2
        z = torch.complex(a[..., :half], a[..., half:])
        th = torch.tensor([s.rope_base ** (-(2 * i) / hd) for i in range(half)], dtype=torch.float64)
        z = z * torch.polar(torch.ones_like(th), pos[:, None, None].double() * th)
        return torch.cat([z.real, z.imag], dim=-1)

    T = len(ids)
    x = t["embed"][torch.from_numpy(ids.astype(np.int64))]
    pos = torch.arange(T)
    for l in range(s.n_layers):
        u = F.rms_norm(x, (s.d_model,), t[f"layers.{l}.attn_norm"], eps=s.rms_eps)
        if s.is_full(l):
            p = f"layers.{l}.fa"
            q = rope(lin(p + ".q", u).view(T, s.fa_q_heads, -1), pos)
            k = rope(lin(p + ".k", u).view(T, s.fa_kv_heads, -1), pos)
            v = lin(p + ".v", u).view(T, s.fa_kv_heads, -1)
            rep = s.fa_q_heads // s.fa_kv_heads
            k, v = k.repeat_interleave(rep, 1), v.repeat_interleave(rep, 1)
            o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1),
                                               v.transpose(0, 1), is_causal=True)
            m = lin(p + ".o", o.transpose(0, 1).reshape(T, -1))
        else:
            p = f"layers.{l}.la"
            q = lin(p + ".q", u).view(T, s.la_heads, -1)
            k = lin(p + ".k", u).view(T, s.la_heads, -1)
            v = lin(p + ".v", u).view(T, s.la_heads, -1)
            g = torch.sigmoid(lin(p + ".g", u))
            S = torch.zeros(s.la_heads, s.la_dk, s.la_dv, dtype=torch.float64)
            outs = []
            for i in range(T):
                S = g[i][:, None, None] * S + torch.einsum("hk,hv->hkv", k[i], v[i])
                outs.append(torch.einsum("hkv,hk->hv", S, q[i]))
            m = lin(p + ".o", torch.stack(outs).reshape(T, -1))
        y = x + m
        w = F.rms_norm(y, (s.d_model,), t[f"layers.{l}.ffn_norm"], eps=s.rms_eps)
        f = f"layers.{l}.ffn"
        x = y + lin(f + ".down", F.silu(lin(f + ".gate", w)) * lin(f + ".up", w))
    return x.numpy()


def test_oracle_forward_matches_independent_torch_formulation(tiny):
    shape, w = tiny
    b = make_batch("tiny-fp32")
    ids = b.tokens_of(0)
    m = O.OracleModel(shape, w.tensors)
    x, hid, _ = m.forward(ids)
    ref = _torch_forward(shape, w.tensors, ids)
    np.testing.assert_allclose(x, ref, rtol=1e-9, atol=1e-10)


def test_float32_mode_agrees_with_float64(tiny):
    shape, w = tiny
    b = make_batch("tiny-fp32")
    r64 = O.prefill_decide(O.OracleModel(shape, w.tensors), b, capture={0: np.arange(128)})
    r32 = O.prefill_decide(O.OracleModel(shape, w.tensors, dtype=np.float32), b,
                           capture={0: np.arange(128)})
    h64, h32 = r64["hidden"][0], r32["hidden"][0]
    for l in range(h64.shape[0]):
        assert np.linalg.norm(h32[l] - h64[l]) / np.linalg.norm(h64[l]) < 1e-5
    for j in r64["probs"]:
        assert np.abs(r32["probs"][j] - r64["probs"][j]).max() < 1e-5


def test_merged_equals_unmerged_for_fp32_storage(tiny):
    shape, w = tiny
    b = make_batch("tiny-fp32")
    a = O.prefill_decide(O.OracleModel(shape, w.tensors), b)
    u = O.prefill_decide(O.OracleModel(shape, w.tensors, lora="unmerged"), b)
    for j in a["probs"]:
        np.testing.assert_allclose(a["probs"][j], u["probs"][j], rtol=1e-10, atol=1e-12)


def test_branch_continuation_equals_plain_forward(tiny):
    shape, w = tiny
    # prefix 100 (not a multiple of 64) + 3 branches of 13, 64, 1 tokens
    b = random_batch(shape.vocab, [100, 13, 64, 1], seed=7, prefix_of=[-1, 0, 0, 0])
    m = O.OracleModel(shape, w.tensors)
    cap = {1: np.arange(13), 2: np.arange(64)}
    plain = O.prefill_decide(m, b, mode="plain", capture=cap)
    cont = O.prefill_decide(m, b, mode="continuation", capture=cap)
    for i in cap:
        np.testing.assert_allclose(cont["hidden"][i], plain["hidden"][i], rtol=1e-9, atol=1e-10)
    for j in plain["probs"]:
        np.testing.assert_allclose(cont["probs"][j], plain["probs"][j], rtol=1e-9, atol=1e-12)


def test_varlen_equals_each_request_alone(tiny):
    shape, w = tiny
    b = random_batch(shape.vocab, [40, 1, 77], seed=3)
    m = O.OracleModel(shape, w.tensors)
    together = O.prefill_decide(m, b)
    for i in range(3):
        x, _, _ = m.forward(b.tokens_of(i))
        for j in np.nonzero(b.q_seq == i)[0]:
            p, _ = m.decide(x[b.q_marker[j]], int(b.q_type[j]), b.options_of(j))
            np.testing.assert_array_equal(p, together["probs"][int(j)])


def test_bf16_merge_effect_is_small():
    """The merged-bf16 model against the unmerged adapter on unrounded base
    weights (the qualification asked for in RFC #114, section 3), on a
    reduced-depth bf16 shape so that it runs in seconds on the CPU."""
    from dataclasses import replace
    shape = replace(shape_of("4b-single-512"), name="bf16-mini", n_layers=4, d_model=256,
                    ffn=512, vocab=2048, la_heads=2, fa_q_heads=2, fa_kv_heads=1, shape_id=77)
    w = make_weights(shape)
    b = random_batch(shape.vocab, [96], seed=11, questions_per_seq=[4])
    a = O.prefill_decide(O.OracleModel(shape, w.tensors), b)
    u = O.prefill_decide(O.OracleModel(shape, w.tensors, lora="unmerged"), b)
    worst = max(np.abs(a["probs"][j] - u["probs"][j]).max() for j in a["probs"])
    assert worst < 0.05


# ------------------------------------------------ planted mistakes (CPU only)
def test_pins_catch_planted_mistakes(monkeypatch):
    """Each mutation of the oracle makes at least one pin fail."""
    import tests.test_oracle_pins as P

    def fails(fn, *args):
        try:
            fn(*args)
        except AssertionError:
            return True
        return False

    real_rope = O.rope_rotate_half
    def rope_wrong_sign(a, pos, base):           # rotation in the wrong direction
        return real_rope(a, -np.asarray(pos), base)
    monkeypatch.setattr(O, "rope_rotate_half", rope_wrong_sign)
    monkeypatch.setattr(P.O, "rope_rotate_half", rope_wrong_sign)
    assert fails(P.test_rope_equals_complex_rotation)
    monkeypatch.undo()

    real_scan = O.la_scan_recurrent
    def scan_no_diagonal(q, k, v, g, S0=None):   # o_t reads S_{t-1} instead of S_t
        o, S = real_scan(q, k, v, g, S0)
        o2 = np.zeros_like(o)
        o2[1:] = o[:-1]
        return o2, S
    monkeypatch.setattr(P.O, "la_scan_recurrent", scan_no_diagonal)
    assert fails(P.test_scan_gate_one_is_causal_linear_attention, scan_no_diagonal)
    monkeypatch.undo()

    real_attn = O.causal_attention
    def attn_no_scale(q, k, v, qp, kp):          # forgets 1/sqrt(hd)
        return real_attn(q * math.sqrt(q.shape[-1]), k, v, qp, kp)
    monkeypatch.setattr(P.O, "causal_attention", attn_no_scale)
    assert fails(P.test_attention_matches_torch_sdpa)
    monkeypatch.undo()

    real_fields = O.decision_fields
    def fields_unnormalised(p, qtype):            # entropy not divided by ln K
        f = real_fields(p, qtype)
        if qtype != O.QTYPE_NOUL:
            f["confidence"] = 1.0 - (1.0 - f["confidence"]) * math.log(len(p))
        return f
    monkeypatch.setattr(P.O, "decision_fields", fields_unnormalised)
    assert fails(P.test_readout_golden_special_cases)
    monkeypatch.undo()

    real_vlp = O.vocab_log_probs
    def vlp_last_chunk_dropped(h, w, E, eps, rows, toks, dtype=np.float64, chunk=16384):
        V = E.shape[0]                           # the denominator loses the ragged last chunk
        keep = V - (V % chunk) if V % chunk else V
        logp, lse = real_vlp(h, w, E, eps, rows, toks, dtype, chunk)
        _, short = real_vlp(h, w, E[:keep], eps, [0], [0], dtype, chunk)
        r = np.asarray(rows)
        return logp + lse[r] - short[r], short
    monkeypatch.setattr(P.O, "vocab_log_probs", vlp_last_chunk_dropped)
    assert fails(P.test_vocab_log_probs_normalise_over_the_whole_vocabulary)
    monkeypatch.undo()

    def vlp_no_final_norm(h, w, E, eps, rows, toks, dtype=np.float64, chunk=16384):
        hn = np.asarray(h, dtype=np.float64) * np.asarray(w)  # gain kept, 1/rms lost
        return real_vlp(hn * 1e6, np.ones(len(w)), E, 0.0, rows, toks, dtype, chunk)
    monkeypatch.setattr(P.O, "vocab_log_probs", vlp_no_final_norm)
    assert fails(P.test_vocab_log_probs_brute_force_loops)
    monkeypatch.undo()

    monkeypatch.undo()

    def gdn_delta_sign(q, k, v, g, beta, S0=None):   # adds beta k k^T S instead of removing it
        T, H, dk = q.shape
        S = np.zeros((H, dk, v.shape[2])) if S0 is None else np.array(S0, dtype=float)
        o = np.zeros((T, H, v.shape[2]))
        for t in range(T):
            kS = np.einsum("hk,hkv->hv", k[t], S)
            S = g[t][:, None, None] * (S + beta[t][:, None, None] * k[t][:, :, None] * kS[:, None, :]) \
                + beta[t][:, None, None] * k[t][:, :, None] * v[t][:, None, :]
            o[t] = np.einsum("hkv,hk->hv", S, q[t])
        return o, S
    monkeypatch.setattr(P.O, "gdn_recurrent", gdn_delta_sign)
    assert fails(P.test_gdn_rewrite_under_one_key)
    monkeypatch.undo()

    real_chunked = O.gdn_chunked
    def gdn_chunk_no_carry(q, k, v, g, beta, S0=None, chunk=64):   # drops the state between chunks
        T = q.shape[0]
        outs = [real_chunked(q[a:a + chunk], k[a:a + chunk], v[a:a + chunk], g[a:a + chunk],
                             beta[a:a + chunk], S0 if a == 0 else None, chunk)[0] for a in range(0, T, chunk)]
        return np.concatenate(outs), None
    monkeypatch.setattr(P.O, "gdn_chunked", gdn_chunk_no_carry)
    assert fails(P.test_gdn_chunked_equals_recurrence, 150, 64)
    monkeypatch.undo()

    real_cand = O.candidate_log_probs
    def cand_over_all_groups(logp, off, grp):     # normalises across questions
        return real_cand(logp, off, np.zeros(len(grp), dtype=np.int64))
    monkeypatch.setattr(P.O, "candidate_log_probs", cand_over_all_groups)
    assert fails(P.test_candidate_log_probs_hand_values)


def test_bf16_activation_mode():
    """act='bf16' rounds matrix-product operands to bf16 (RFC #114 section 1:
    BF16 inference); its drift from exact arithmetic is of bf16 size -- not
    zero, and far below O(1)."""
    from dataclasses import replace
    shape = replace(shape_of("4b-single-512"), name="bf16-mini", n_layers=4, d_model=256,
                    ffn=512, vocab=2048, la_heads=2, fa_q_heads=2, fa_kv_heads=1, shape_id=78)
    w = make_weights(shape)
    om = O.OracleModel(shape, w.tensors, act="bf16")
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 0.02, -3.3])
    np.testing.assert_array_equal(om._a(x), O.bf16_bits_to_float(O.round_to_bf16_bits(x)))
    assert O.OracleModel(shape, w.tensors)._a(x) is x
    b = random_batch(shape.vocab, [80], seed=2, questions_per_seq=[3])
    cap = {0: np.arange(80)}
    hb = O.prefill_decide(om, b, capture=cap)["hidden"][0]
    hx = O.prefill_decide(O.OracleModel(shape, w.tensors), b, capture=cap)["hidden"][0]
    drift = [np.linalg.norm(hb[l] - hx[l]) / np.linalg.norm(hx[l]) for l in range(1, 5)]
    assert all(1e-4 < d < 3e-2 for d in drift), drift


def test_token_log_probs_match_torch_log_softmax(tiny):
    """The model-level features against torch's log_softmax over the full
    tied-embedding logits of the independent torch formulation's rows."""
    shape, w = tiny
    ids = make_batch("tiny-fp32").tokens_of(0)
    m = O.OracleModel(shape, w.tensors)
    x, _, _ = m.forward(ids)
    F = torch.nn.functional
    xt = torch.from_numpy(_torch_forward(shape, w.tensors, ids))
    hn = F.rms_norm(xt, (shape.d_model,), torch.from_numpy(w.tensors["final_norm"].astype(np.float64)),
                    eps=shape.rms_eps)
    ref = F.log_softmax(hn @ torch.from_numpy(w.tensors["embed"].astype(np.float64)).T, dim=-1).numpy()
    rows = np.arange(len(ids) - 1)
    logp, lse = m.token_log_probs(x, rows, ids[1:])
    np.testing.assert_allclose(logp, ref[rows, ids[1:]], rtol=1e-9, atol=1e-9)
    assert lse.shape == (len(ids),)


def _torch_gdn_forward(shape, tensors, ids):
    """Independent PyTorch formulation of a Gated DeltaNet hybrid (float64):
    F.conv1d for the short convolution, the delta rule as a token loop."""
    F = torch.nn.functional
    t = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in tensors.items()}
    s = shape
    sc = s.lora_alpha / s.lora_rank

    def lin(name, x):
        y = F.linear(x, t[name])
        if name + ".lora_A" in t:
            y = y + sc * F.linear(F.linear(x, t[name + ".lora_A"]), t[name + ".lora_B"])
        return y

    def rope(a, pos):
        hd = a.shape[-1]
        half = hd // 2
        z = torch.complex(a[..., :half], a[..., half:])
        th = torch.tensor([s.rope_base ** (-(2 * i) / hd) for i in range(half)], dtype=torch.float64)
        z = z * torch.polar(torch.ones_like(th), pos[:, None, None].double() * th)
        return torch.cat([z.real, z.imag], dim=-1)

    T = len(ids)
    H, dk, dv = s.la_heads, s.la_dk, s.la_dv
    x = t["embed"][torch.from_numpy(ids.astype(np.int64))]
    pos = torch.arange(T)
    for l in range(s.n_layers):
        u = F.rms_norm(x, (s.d_model,), t[f"layers.{l}.attn_norm"], eps=s.rms_eps)
        if s.is_full(l):
            p = f"layers.{l}.fa"
            q = rope(lin(p + ".q", u).view(T, s.fa_q_heads, -1), pos)
            k = rope(lin(p + ".k", u).view(T, s.fa_kv_heads, -1), pos)
            v = lin(p + ".v", u).view(T, s.fa_kv_heads, -1)
            rep = s.fa_q_heads // s.fa_kv_heads
            k, v = k.repeat_interleave(rep, 1), v.repeat_interleave(rep, 1)
            o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1),
                                               v.transpose(0, 1), is_causal=True)
            m = lin(p + ".o", o.transpose(0, 1).reshape(T, -1))
        else:
            p = f"layers.{l}.la"
            pre = torch.cat([lin(p + ".q", u), lin(p + ".k", u), lin(p + ".v", u)], dim=1)     # [T, C]
            w = t[p + ".conv"]                                                              # [C, 4]
            y = F.silu(F.conv1d(F.pad(pre.T[None], (3, 0)), w[:, None, :], groups=w.shape[0])[0].T)
            nrm = lambda a: a / torch.sqrt((a * a).sum(-1, keepdim=True) + 1e-6)
            q = nrm(y[:, :H * dk].view(T, H, dk)) / dk ** 0.5
            k = nrm(y[:, H * dk:2 * H * dk].view(T, H, dk))
            v = y[:, 2 * H * dk:].view(T, H, dv)
            g = torch.sigmoid(lin(p + ".g", u))
            beta = torch.sigmoid(lin(p + ".b", u))
            S = torch.zeros(H, dk, dv, dtype=torch.float64)
            outs = []
            eye = torch.eye(dk, dtype=torch.float64)
            for i in range(T):
                P = eye[None] - beta[i][:, None, None] * torch.einsum("hk,hj->hkj", k[i], k[i])
                S = g[i][:, None, None] * torch.bmm(P, S) + beta[i][:, None, None] * torch.einsum("hk,hv->hkv", k[i], v[i])
                outs.append(torch.einsum("hkv,hk->hv", S, q[i]))
            m = lin(p + ".o", torch.stack(outs).reshape(T, -1))
        y2 = x + m
        wn = F.rms_norm(y2, (s.d_model,), t[f"layers.{l}.ffn_norm"], eps=s.rms_eps)
        f = f"layers.{l}.ffn"
        x = y2 + lin(f + ".down", F.silu(lin(f + ".gate", wn)) * lin(f + ".up", wn))
    return x.numpy()


def test_gdn_oracle_matches_independent_torch_formulation():
    from dataclasses import replace
    shape = replace(shape_of("tiny-fp32"), name="tiny-gdn", la_kind="gdn", shape_id=9)
    w = make_weights(shape)
    ids = make_batch("tiny-fp32").tokens_of(0)[:70]
    x, _, _ = O.OracleModel(shape, w.tensors).forward(ids)
    np.testing.assert_allclose(x, _torch_gdn_forward(shape, w.tensors, ids), rtol=1e-9, atol=1e-10)


def test_gdn_branch_continuation_equals_plain_forward():
    """A branch continued from the prefix's state and convolution history is
    the plain forward of prefix + branch ([rfc114] section 5: the snapshot
    holds the recurrent state and the convolution history)."""
    from dataclasses import replace
    shape = replace(shape_of("tiny-fp32"), name="tiny-gdn", la_kind="gdn", shape_id=9)
    w = make_weights(shape)
    m = O.OracleModel(shape, w.tensors)
    b = random_batch(shape.vocab, [67, 2, 40], seed=3, prefix_of=[-1, 0, 0], questions_per_seq=[0, 1, 2])
    r1 = O.prefill_decide(m, b, mode="plain")
    r2 = O.prefill_decide(m, b, mode="continuation")
    for j in r1["probs"]:
        np.testing.assert_allclose(r2["probs"][j], r1["probs"][j], rtol=1e-10, atol=1e-12)
