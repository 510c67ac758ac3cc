"""Plain numpy oracle of the prefill-only decision path (test infrastructure).

Every function states the passage of the pages it follows.  Page names used:
  [omni-readme]  System1-Omni README
  [rfc114]       RFC #114, "Native Rust/CUDA support for OmniJev-4B v1.1"
  [rfc114-plan]  RFC #114, comment "Plan: native OmniJev-4B v1.1"
  [sys1rust]     sys1rust README
  [cua-issue]    "[New Model]: Support Cua-S1 4B 0.2", issue #10
Readings taken where the pages are silent (tags used below):
  (R1)  linear attention is the stated stand-in S_t = g_t S_{t-1} + k_t v_t^T,
        o_t = S_t^T q_t: update first, then read, so o_t sees token t.  No
        feature map, q/k norm, 1/sqrt(dk), short conv, delta rule or output
        gate (the pages name Gated DeltaNet but print no equations).
  (R2)  one decay gate per (token, head): g = sigmoid(u . w_g[h]), no bias.
  (R3)  the state is zero at a sequence start; a branch starts from its
        prefix's final state ([rfc114] section 5).
  (R4)  layer l is full attention iff l % full_every == full_every - 1
        (3 linear then 1 full; the tiny shape alternates).
  (R5)  packed sequences are independent.
  (R6)  pre-norm residual blocks, RMSNorm before the mixer and the FFN, one
        final RMSNorm before the readout.
  (R7)  RMSNorm eps 1e-6 everywhere, gains initialised to one.
  (R8)  grouped-query attention with contiguous groups, scale 1/sqrt(hd),
        causal mask including the diagonal, no biases.
  (R9)  rotate-half RoPE over the whole head dim, base 10000; positions
        restart at 0 per sequence; branch token j sits at position P + j.
  (R10) SwiGLU FFN, no biases anywhere.
  (R11) choice ties go to the lowest option index.
  (R12) score levels are numbered 0..K-1 in caller order.
  (R13) noul options are ordered [yes, no].
  (R14) the readout softmax runs over the question's K option logits only, no
        temperature or bias.
  (R15) LoRA targets: q, k, v, o of both mixer kinds (+ FFN gate, up, down on
        the 4B/27B shapes); the decay-gate projection is not adapted.
  (R23) Gated DeltaNet (the layer the pages run, replacing the stand-in when
        a shape asks for it): short causal depthwise convolution of width 4
        on the q, k and v projections, then SiLU; q and k L2-normalised per
        head (eps 1e-6 inside the root) and q scaled by 1/sqrt(dk); the gate
        g of R2 as the decay; one write strength beta = sigmoid(u . w_b) per
        (token, head); the gated delta update; no output gate or norm.
  (R21) a feature candidate scores the sum of its tokens' full-vocabulary
        log-probabilities, normalised by a log-softmax across the candidates
        of its question (the six-feature composition on top is not built).
"""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

QTYPE_CHOICE, QTYPE_SCORE, QTYPE_NOUL = 0, 1, 2


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------
def bf16_bits_to_float(bits, dtype=np.float64):
    """Decode bfloat16 bit patterns (uint16): a bf16 value is the top half of
    the float32 with the same sign, exponent and leading mantissa bits."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype, copy=False)


def round_to_bf16_bits(x):
    """Round float64 values to bfloat16, to nearest with ties to even, in one
    step (no intermediate float32 rounding).  A float64 keeps 52 explicit
    mantissa bits and a bf16 keeps 7, so 45 low bits are rounded away on the
    float64 bit pattern; the 8-significant-bit result is exactly a float32,
    whose top 16 bits are the bf16 pattern.  Inputs are finite and inside the
    float32 normal range."""
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = ((u + lsb + np.uint64((1 << 44) - 1)) >> np.uint64(45)) << np.uint64(45)
    f32 = u.view(np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------
def rms_norm(x, w, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w.  (R6, R7):
    the pages name Qwen3.5-family backbones ([omni-readme], directory table;
    [cua-issue], model request), whose blocks are pre-norm with RMSNorm."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def rope_rotate_half(a, pos, base):
    """Rotary position embedding, rotate-half pairing (R9): for i < hd/2 the
    pair (a_i, a_{i+hd/2}) is rotated by angle pos * base^(-2i/hd).
    a: [T, H, hd]; pos: [T] integer positions.  Angles are formed in float64."""
    T, H, hd = a.shape
    half = hd // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang).astype(a.dtype)[:, None, :]
    s = np.sin(ang).astype(a.dtype)[:, None, :]
    a1, a2 = a[..., :half], a[..., half:]
    return np.concatenate([a1 * c - a2 * s, a2 * c + a1 * s], axis=-1)


def la_scan_recurrent(q, k, v, g, S0=None):
    """Gated linear attention, the recurrence itself, one token at a time:
        S_t = g_t * S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
    per head, with S a [dk, dv] state and g_t a scalar per (token, head) (R1,
    R2).  The state is float64 here, at least the fp32 the pages require for
    the recurrent state ([rfc114] section 5).  S0 is the initial state (zero
    at a sequence start, the prefix's final state for a branch).
    q, k: [T, H, dk]; v: [T, H, dv]; g: [T, H].  Returns (o [T, H, dv], S_T)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((H, dk, dv), dtype=q.dtype) if S0 is None else np.array(S0, dtype=q.dtype)
    o = np.zeros((T, H, dv), dtype=q.dtype)
    for t in range(T):
        S = g[t][:, None, None] * S + k[t][:, :, None] * v[t][:, None, :]
        o[t] = np.einsum("hkv,hk->hv", S, q[t])
    return o, S


def la_scan_unrolled(q, k, v, g, S0=None):
    """The same recurrence in closed form (unrolled), computed with matmuls:
        o_t = sum_{s<=t} exp(G_t - G_s) (q_t . k_s) v_s + exp(G_t) S0^T q_t
        S_T = sum_s exp(G_{T-1} - G_s) k_s v_s^T + exp(G_{T-1}) S0
    with G_t = sum_{r<=t} log g_r.  Decays are formed as exp of a difference,
    never as a ratio of products (products of many gates underflow).  G and the
    decay factors are formed in float64 in every mode.  Exact reformulation of
    la_scan_recurrent; the tests check one against the other."""
    T, H, dk = q.shape
    dv = v.shape[2]
    dt = q.dtype
    S_init = np.zeros((H, dk, dv), dtype=dt) if S0 is None else np.asarray(S0, dtype=dt)
    o = np.zeros((T, H, dv), dtype=dt)
    S_fin = np.array(S_init, copy=True)
    if T == 0:
        return o, S_fin
    # a gate of exactly 0 is clamped to 1e-300 so that every log is finite;
    # the decays it produces are below 1e-300 and vanish in the sums.
    G = np.cumsum(np.log(np.maximum(np.asarray(g, dtype=np.float64), 1e-300)), axis=0)
    tri = np.tril(np.ones((T, T), dtype=bool))
    for h in range(H):
        Gh = G[:, h]
        D = np.where(tri, np.exp(np.minimum(Gh[:, None] - Gh[None, :], 0.0)), 0.0)
        A = (q[:, h, :] @ k[:, h, :].T) * D.astype(dt)
        o[:, h, :] = A @ v[:, h, :] + np.exp(Gh).astype(dt)[:, None] * (q[:, h, :] @ S_init[h])
        w_last = np.exp(Gh[-1] - Gh).astype(dt)                          # [T]
        S_fin[h] = (k[:, h, :] * w_last[:, None]).T @ v[:, h, :] + np.exp(Gh[-1]).astype(dt) * S_init[h]
    return o, S_fin


def la_scan_segmented(q, k, v, g, S0=None, segment=512):
    """The recurrence over consecutive segments of the sequence, each in the
    unrolled form, the state at a segment's end being the next segment's
    initial state -- the state summarises everything before it, which is also
    what lets a branch continue from a prefix ([rfc114] section 5).  Bounds
    the unrolled form's T x T decay matrix for long sequences."""
    T, H, _ = q.shape
    o = np.zeros((T, H, v.shape[2]), dtype=q.dtype)
    S = S0
    if T == 0:
        return la_scan_unrolled(q, k, v, g, S0)
    for a in range(0, T, segment):
        b = min(T, a + segment)
        o[a:b], S = la_scan_unrolled(q[a:b], k[a:b], v[a:b], g[a:b], S)
    return o, S


def l2_normalize(x, eps=1e-6):
    """x / sqrt(sum(x^2) + eps) over the last axis (the q / k normalisation of
    Gated DeltaNet; the eps is reading R23)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def silu(x):
    return x / (1.0 + np.exp(-x))


def causal_conv_silu(x, w, hist=None):
    """Depthwise causal convolution over time, then SiLU (the short
    convolution of Gated DeltaNet, R23):
        y[t, c] = silu(sum_{j < W} w[c, j] * x[t - (W - 1) + j, c])
    so w[c, W - 1] weighs the current token.  Rows before the sequence come
    from hist [W - 1, C] (the last rows of a prefix, for a branch) or are
    zero.  x: [T, C]; w: [C, W].  Returns (y [T, C], the last W - 1 rows of
    the extended input, the history a continuation needs)."""
    T, C = x.shape
    W = w.shape[1]
    h = np.zeros((W - 1, C), dtype=x.dtype) if hist is None else np.asarray(hist, dtype=x.dtype)
    ext = np.concatenate([h, x], axis=0)
    y = np.zeros_like(x)
    for j in range(W):
        y += w[:, j][None, :] * ext[j:j + T]
    return silu(y), ext[T:]


def gdn_recurrent(q, k, v, g, beta, S0=None):
    """Gated delta rule, token by token (Yang, Kautz, Hatamizadeh, "Gated
    Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025, the gated
    delta update), written for a [dk, dv] state read as S^T q:
        S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
        o_t = S_t^T q_t.
    g_t in (0, 1] decays the state, beta_t in (0, 1) is the write strength;
    with a unit key and beta = 1 the state then returns exactly v_t for k_t.
    q, k: [T, H, dk]; v: [T, H, dv]; g, beta: [T, H].  Returns (o, S_T)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((H, dk, dv), dtype=q.dtype) if S0 is None else np.array(S0, dtype=q.dtype)
    o = np.zeros((T, H, dv), dtype=q.dtype)
    for t in range(T):
        kS = np.einsum("hk,hkv->hv", k[t], S)                       # k_t^T S_{t-1}
        S = g[t][:, None, None] * (S - beta[t][:, None, None] * k[t][:, :, None] * kS[:, None, :]) \
            + beta[t][:, None, None] * k[t][:, :, None] * v[t][:, None, :]
        o[t] = np.einsum("hkv,hk->hv", S, q[t])
    return o, S


def gdn_chunked(q, k, v, g, beta, S0=None, chunk=64):
    """The gated delta rule over chunks of `chunk` tokens in the WY form
    (Yang et al., "Parallelizing Linear Transformers with the Delta Rule over
    Sequence Length", NeurIPS 2024, extended with the gate as in the Gated
    DeltaNet paper).  Writing S_t = g_t S_{t-1} + k_t u_t^T with
    u_t = beta_t (v_t - g_t S_{t-1}^T k_t), and, inside a chunk starting from
    S_0, gamma_t = prod_{j <= t} g_j:
        (I + L) U = diag(beta) V - diag(beta gamma) K S_0,
            L[t, i] = beta_t (gamma_t / gamma_i) k_t . k_i  for i < t,
        O   = diag(gamma) Q S_0 + ((Q K^T) * M) U,  M[t, i] = gamma_t / gamma_i, i <= t,
        S_C = gamma_C S_0 + K^T diag(gamma_C / gamma) U.
    The unit lower-triangular system is solved by forward substitution.
    Gamma ratios are formed as exp of differences of cumulative logs (each
    at most 1).  An exact reformulation of gdn_recurrent (the tests check one
    against the other).  Returns (o, S_T)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    dt = q.dtype
    S = np.zeros((H, dk, dv), dtype=dt) if S0 is None else np.array(S0, dtype=dt)
    o = np.zeros((T, H, dv), dtype=dt)
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        C = b - a
        G = np.cumsum(np.log(np.maximum(np.asarray(g[a:b], dtype=np.float64), 1e-300)), axis=0)   # [C, H]
        tri_s = np.tril(np.ones((C, C), dtype=bool), -1)
        tri = np.tril(np.ones((C, C), dtype=bool))
        for h in range(H):
            Kc, Vc, Qc = k[a:b, h], v[a:b, h], q[a:b, h]
            Gh = G[:, h]
            bt = np.asarray(beta[a:b, h], dtype=dt)
            R = np.exp(np.minimum(Gh[:, None] - Gh[None, :], 0.0))                     # gamma_t / gamma_i
            L = np.where(tri_s, bt[:, None] * R * (Kc @ Kc.T), 0.0).astype(dt)
            rhs = bt[:, None] * Vc - (bt * np.exp(Gh))[:, None] * (Kc @ S[h])
            U = np.zeros((C, dv), dtype=dt)
            for t in range(C):
                U[t] = rhs[t] - L[t, :t] @ U[:t]
            M = np.where(tri, R, 0.0).astype(dt)
            o[a:b, h] = np.exp(Gh)[:, None] * (Qc @ S[h]) + ((Qc @ Kc.T) * M) @ U
            S[h] = np.exp(Gh[-1]) * S[h] + (Kc * np.exp(Gh[-1] - Gh)[:, None]).T @ U
    return o, S


def causal_attention(q, k, v, q_pos, k_pos):
    """Causal softmax attention, the definition: for query head h with kv head
    h // (Hq / Hkv) (grouped, contiguous groups, R8),
        o_t = sum_{s : pos_s <= pos_t} softmax_s(q_t . k_s / sqrt(hd)) v_s.
    The diagonal is included.  q: [Tq, Hq, hd]; k, v: [Tk, Hkv, hd]."""
    Tq, Hq, hd = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    o = np.zeros((Tq, Hq, v.shape[2]), dtype=q.dtype)
    if Tq == 0:
        return o
    mask = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    scale = 1.0 / math.sqrt(hd)
    for h in range(Hq):
        kv = h // grp
        s = (q[:, h, :] @ k[:, kv, :].T) * scale
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ v[:, kv, :]
    return o


def swiglu(u, w_gate, w_up, w_down):
    """SwiGLU FFN (R10): down( silu(u W_gate^T) * (u W_up^T) ), silu(a) = a sigmoid(a)."""
    a = u @ w_gate.T
    b = u @ w_up.T
    return (a * sigmoid(a) * b) @ w_down.T


def lora_merge(w, a, b, alpha, rank):
    """Merged LoRA weight W' = W + (alpha / r) B A ([rfc114] section 3 asks for
    the merge at load; [cua-issue] first plan comment: merged at load).
    w: [out, in]; a: [r, in]; b: [out, r]."""
    return w + (alpha / rank) * (b @ a)


def softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def decision_fields(p, qtype):
    """Answer fields from option probabilities p (caller order), after
    [sys1rust] "Try it": choice is the most likely option (lowest index on an
    exact tie, R11); score is the expected level, levels numbered 0..K-1 in
    caller order (R12), so it can fall between levels; noul is P(yes) with
    options ordered [yes, no]; answer_confidence is the largest probability;
    for choice and score, confidence is 1 minus the normalised entropy
    (0 for an even split, 1 for a one-hot); for noul, confidence equals
    answer_confidence.  entropy_confidence = 1 - H(p)/ln K for every type.
    0 ln 0 is taken as 0."""
    p = np.asarray(p, dtype=np.float64)
    K = len(p)
    choice = int(np.argmax(p))
    score = float(np.dot(np.arange(K, dtype=np.float64), p))
    noul = float(p[0])
    ans = float(p.max())
    nz = p[p > 0]
    H = float(-(nz * np.log(nz)).sum())
    ent = float(min(1.0, max(0.0, 1.0 - H / math.log(K))))
    conf = ans if qtype == QTYPE_NOUL else ent
    return {"choice": choice, "score": score, "noul": noul,
            "answer_confidence": ans, "confidence": conf,
            "entropy_confidence": ent}


def readout(h_row, w_final, e_rows, eps, qtype):
    """Decision readout of one question: final RMSNorm of the marker row,
    option logits z_k = h . E[opt_k] against the tied embedding rows, softmax
    over the K option logits only ([cua-issue] first plan comment: the answer
    is read from the option logits of a single pass; [rfc114-plan]: the head
    stays bf16 and is cast to fp32 before the softmax -- here the whole
    readout runs in the oracle's float type).  Returns (p, fields)."""
    h = rms_norm(h_row[None, :], w_final, eps)[0]
    z = e_rows @ h
    p = softmax(z)
    return p, decision_fields(p, qtype)


def vocab_log_probs(h_rows, w_final, embed, eps, rows, tokens, dtype=np.float64, chunk=16384):
    """Full-vocabulary token log-probabilities (the language-model features of
    [rfc114] section 4, note under the semantics table: token log-probabilities
    normalised over the whole vocabulary, with the vocabulary work done in
    bounded chunks; [rfc114-plan]: the log-softmax runs over every row of the
    tied embedding, with the head's logits taken to fp32 first -- here the
    oracle's float type).

    h_rows [R, d]: residual-stream rows before the final norm.  embed: the raw
    tied embedding [V, d] (bf16 bit patterns or floats), decoded `chunk` rows
    at a time so that no [V, d] float copy is held.  Target n is token
    tokens[n] read from row rows[n].  With hn = RMSNorm(h; w_final) and
    z[r, v] = hn[r] . E[v] for every v in [0, V):
        lse[r]  = log sum_v exp(z[r, v])
        logp[n] = z[rows[n], tokens[n]] - lse[rows[n]]
    (the log-sum-exp is evaluated as m + log sum exp(z - m) with m the row
    maximum, the same number).  Returns (logp [n], lse [R])."""
    hn = rms_norm(np.asarray(h_rows, dtype=dtype), np.asarray(w_final, dtype=dtype), eps)
    V = embed.shape[0]
    z = np.empty((hn.shape[0], V), dtype=dtype)
    for v0 in range(0, V, chunk):
        e = embed[v0:v0 + chunk]
        e = bf16_bits_to_float(e, dtype) if e.dtype == np.uint16 else e.astype(dtype)
        z[:, v0:v0 + e.shape[0]] = hn @ e.T
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    rows = np.asarray(rows, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    return z[rows, tokens] - lse[rows], lse


def candidate_log_probs(logp, cand_offsets, cand_group):
    """Candidate scores and their normalisation across the candidates of one
    question ([rfc114] section 4, note under the semantics table: the token
    log-probabilities are normalised over the vocabulary and then again across
    the candidates of the same question).  Reading (R21): a candidate owns the
    targets cand_offsets[c] .. cand_offsets[c+1]-1 and scores the sum of their
    log-probabilities (the log-probability of its whole token string; an empty
    candidate scores 0); candidates with equal cand_group form one question,
    normalised as  norm[c] = lp[c] - log sum_{c' in group(c)} exp(lp[c']).
    Returns (lp [C], norm [C])."""
    logp = np.asarray(logp, dtype=np.float64)
    off = np.asarray(cand_offsets, dtype=np.int64)
    grp = np.asarray(cand_group, dtype=np.int64)
    C = len(grp)
    lp = np.array([logp[off[c]:off[c + 1]].sum() for c in range(C)], dtype=np.float64)
    norm = np.empty(C, dtype=np.float64)
    for g in np.unique(grp):
        sel = np.nonzero(grp == g)[0]
        m = lp[sel].max()
        norm[sel] = lp[sel] - (m + math.log(np.exp(lp[sel] - m).sum()))
    return lp, norm


# --------------------------------------------------------------------------
# the hybrid decoder
# --------------------------------------------------------------------------
class OracleModel:
    """Hybrid decoder with merged LoRA, evaluated in `dtype` (float64 default).

    Weights arrive as the generator's raw tensors: bf16 bit patterns (uint16)
    or float32.  For a bf16 model each LoRA target is merged in float64 and
    rounded once to bf16, the merged storage the pages describe ([rfc114]
    section 1: adapter merged into BF16 weights); for an fp32 model the merge
    is kept exact.  With lora="unmerged" the adapter is applied at run time as
    W x + (alpha/r) B (A x) on the unrounded base (the comparison [rfc114]
    section 3 asks for).  Weights are decoded to `dtype` at each use unless
    keep_decoded=True."""

    def __init__(self, shape, tensors, dtype=np.float64, lora="merged",
                 keep_decoded=False, threads=0, act="exact"):
        self.s = shape
        self.dtype = np.dtype(dtype)
        # act="bf16": the operands of every matrix product the method runs in
        # bf16 are bf16 values (see `_a`); act="exact": no activation rounding.
        if act not in ("exact", "bf16"):
            raise ValueError(act)
        self.act = act
        self.lora = lora
        self.bf16 = shape.dtype == "bf16"
        self.keep = keep_decoded
        self._raw = tensors
        self._store = {}
        self._dec = {}
        self.scale = shape.lora_alpha / shape.lora_rank
        targets = [n[:-len(".lora_A")] for n in tensors if n.endswith(".lora_A")]
        if lora == "merged":
            def job(name):
                self._store[name] = self._merge(name)
            if threads <= 0:
                threads = 8
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(job, targets))
        self.targets = set(targets)

    # -- weights ---------------------------------------------------------
    def _to_float(self, raw, dtype=None):
        dtype = dtype or self.dtype
        if raw.dtype == np.uint16:
            return bf16_bits_to_float(raw, dtype)
        return raw.astype(dtype, copy=False)

    def _merge(self, name):
        w = self._to_float(self._raw[name], np.float64)
        a = self._to_float(self._raw[name + ".lora_A"], np.float64)
        b = self._to_float(self._raw[name + ".lora_B"], np.float64)
        m = lora_merge(w, a, b, self.s.lora_alpha, self.s.lora_rank)
        return round_to_bf16_bits(m) if self.bf16 else m

    def merged_storage(self, name):
        """The merged weight as stored (bf16 bits or float64)."""
        return self._store.get(name, self._raw[name])

    def W(self, name):
        if name in self._dec:
            return self._dec[name]
        w = self._to_float(self._store[name] if name in self._store else self._raw[name])
        if self.keep:
            self._dec[name] = w
        return w

    def _a(self, x):
        """Activation operand of a bf16 matrix product.  The pages fix the
        method's precision as BF16 inference ([rfc114] section 1; [cua-issue]
        timing comments, bfloat16) with an FP32 recurrent state ([rfc114]
        section 5) and an FP32 head ([rfc114-plan]).  In act="bf16" mode the
        operands of the bf16 matrix products -- the input of every projection
        (normalised activations, mixer output, SwiGLU output) and the q, k, v
        operands of attention and of the recurrence -- are rounded to bf16
        (nearest, ties to even); accumulation, norms, the residual stream, the
        state, the softmax and the readout stay in the oracle's float type."""
        if self.act != "bf16":
            return x
        return bf16_bits_to_float(round_to_bf16_bits(x), x.dtype)

    def proj(self, name, u):
        """u W^T, with the LoRA term added at run time in unmerged mode."""
        y = u @ self.W(name).T
        if self.lora == "unmerged" and name in self.targets:
            a = self._to_float(self._raw[name + ".lora_A"])
            b = self._to_float(self._raw[name + ".lora_B"])
            y = y + self.scale * ((u @ a.T) @ b.T)
        return y

    def embed(self, ids):
        return self._to_float(self._raw["embed"][np.asarray(ids)])

    # -- mixers ----------------------------------------------------------
    def _linear(self, l, u, S0):
        if self.s.la_kind == "gdn":
            return self._gdn(l, u, S0)
        s = self.s
        T = u.shape[0]
        p = f"layers.{l}.la"
        u = self._a(u)
        q = self._a(self.proj(p + ".q", u).reshape(T, s.la_heads, s.la_dk))
        k = self._a(self.proj(p + ".k", u).reshape(T, s.la_heads, s.la_dk))
        v = self._a(self.proj(p + ".v", u).reshape(T, s.la_heads, s.la_dv))
        g = sigmoid(self.proj(p + ".g", u))           # (R2) one gate per head
        o, S = la_scan_segmented(q, k, v, g, S0)
        return self.proj(p + ".o", self._a(o.reshape(T, s.la_heads * s.la_dv))), S

    def _gdn(self, l, u, cache):
        """Gated DeltaNet mixer (R23): projections q | k | v (the channels of
        one depthwise causal convolution of width 4, then SiLU), the decay gate
        g = sigmoid(u . w_g) and the write strength beta = sigmoid(u . w_b) per
        head; q and k L2-normalised per head, q scaled by 1/sqrt(dk); the gated
        delta rule (chunked WY form); the out-projection.  cache is None or
        (state, the last 3 pre-convolution rows) of a prefix; returns the
        same pair for this sequence's end."""
        s = self.s
        T = u.shape[0]
        H, dk, dv = s.la_heads, s.la_dk, s.la_dv
        p = f"layers.{l}.la"
        u = self._a(u)
        pre = np.concatenate([self.proj(p + ".q", u), self.proj(p + ".k", u), self.proj(p + ".v", u)], axis=1)
        S0, hist = (None, None) if cache is None else cache
        y, hist_out = causal_conv_silu(pre, self.W(p + ".conv"), hist)
        q = l2_normalize(y[:, :H * dk].reshape(T, H, dk)) / math.sqrt(dk)
        k = l2_normalize(y[:, H * dk:2 * H * dk].reshape(T, H, dk))
        v = y[:, 2 * H * dk:].reshape(T, H, dv)
        g = sigmoid(self.proj(p + ".g", u))
        beta = sigmoid(self.proj(p + ".b", u))
        o, S = gdn_chunked(self._a(q), self._a(k), self._a(v), g, beta, S0)
        return self.proj(p + ".o", self._a(o.reshape(T, H * dv))), (S, hist_out)

    def _full(self, l, u, pos, prefix):
        s = self.s
        T = u.shape[0]
        p = f"layers.{l}.fa"
        u = self._a(u)
        q = self._a(rope_rotate_half(self.proj(p + ".q", u).reshape(T, s.fa_q_heads, s.fa_head_dim),
                                     pos, s.rope_base))
        k = self._a(rope_rotate_half(self.proj(p + ".k", u).reshape(T, s.fa_kv_heads, s.fa_head_dim),
                                     pos, s.rope_base))
        v = self._a(self.proj(p + ".v", u).reshape(T, s.fa_kv_heads, s.fa_head_dim))
        if prefix is not None:
            pk, pv, ppos = prefix
            k = np.concatenate([pk, k], axis=0)
            v = np.concatenate([pv, v], axis=0)
            kpos = np.concatenate([ppos, pos])
        else:
            kpos = pos
        o = causal_attention(q, k, v, pos, kpos)
        return self.proj(p + ".o", self._a(o.reshape(T, s.fa_q_heads * s.fa_head_dim))), (k, v, kpos)

    # -- forward ---------------------------------------------------------
    def forward(self, ids, start_pos=0, cache=None, want_cache=False, capture_rows=None,
                n_layers=None):
        """Forward over one sequence.  Returns (x_final [T, d], hidden, cache):
        hidden[l] = residual stream after the embedding (l = 0) and after
        layer l (l >= 1) at capture_rows (all rows if None); cache holds each
        linear layer's final state and each full layer's keys/values, so that
        a continuation can start from it ([rfc114] section 5: snapshot of the
        full-attention KV and the recurrent state; every branch starts from
        the same snapshot).  n_layers < all runs only the first layers (used
        to time a bounded sample)."""
        s = self.s
        T = len(ids)
        pos = start_pos + np.arange(T, dtype=np.int64)
        x = self.embed(ids)
        rows = slice(None) if capture_rows is None else np.asarray(capture_rows)
        hidden = [x[rows].copy()]
        out_cache = {"la": {}, "fa": {}, "len": start_pos + T}
        for l in range(s.n_layers if n_layers is None else n_layers):
            u = rms_norm(x, self.W(f"layers.{l}.attn_norm"), s.rms_eps)
            if s.is_full(l):
                prefix = None if cache is None else cache["fa"][l]
                m, kv = self._full(l, u, pos, prefix)
                if want_cache:
                    out_cache["fa"][l] = kv
            else:
                S0 = None if cache is None else cache["la"][l]
                m, S = self._linear(l, u, S0)
                if want_cache:
                    out_cache["la"][l] = S
            y = x + m
            v = rms_norm(y, self.W(f"layers.{l}.ffn_norm"), s.rms_eps)
            f = f"layers.{l}.ffn"
            x = y + self._ffn(f, v)
            hidden.append(x[rows].copy())
        return x, hidden, (out_cache if want_cache else None)

    def _ffn(self, f, v):
        v = self._a(v)
        a = self.proj(f + ".gate", v)
        b = self.proj(f + ".up", v)
        return self.proj(f + ".down", self._a(a * sigmoid(a) * b))

    def decide(self, x_row, qtype, option_ids):
        e = self.embed(option_ids)
        return readout(x_row, self.W("final_norm"), e, self.s.rms_eps, qtype)

    def token_log_probs(self, x_rows, rows, tokens):
        """vocab_log_probs over this model's final norm and tied embedding;
        x_rows are final residual-stream rows.  Returns (logp, lse)."""
        return vocab_log_probs(x_rows, self.W("final_norm"), self._raw["embed"], self.s.rms_eps,
                               rows, tokens, dtype=self.dtype)


def prefill_decide(model, batch, mode="plain", capture=None, seqs=None):
    """Answer every question of `batch` (an s1_workloads.Batch).

    Sequences are independent (R5: nothing crosses a sequence boundary).  A
    branch (prefix_of[i] >= 0) is, by definition, the plain forward over
    prefix + suffix restricted to its suffix rows (mode="plain");
    mode="continuation" runs each prefix once and continues every branch from
    its cache, which [rfc114-plan] states equals the plain forward up to
    rounding (checked by the tests).  capture maps a sequence index to rows
    (within that sequence) whose residual stream is returned per layer.
    seqs restricts the work to the listed sequences (questions elsewhere are
    skipped).  Returns {"probs": {j: p}, "fields": {j: dict},
    "hidden": {i: [n_layers + 1, rows, d]}}."""
    capture = capture or {}
    todo = range(batch.n_seqs) if seqs is None else seqs
    probs, fields, hidden = {}, {}, {}
    prefix_cache = {}
    is_prefix = set(int(p) for p in batch.prefix_of if p >= 0)
    for i in todo:
        ids = batch.tokens_of(i)
        pidx = int(batch.prefix_of[i])
        rows = capture.get(i)
        if pidx < 0:
            keep = mode != "plain" and i in is_prefix
            x, hid, c = model.forward(ids, capture_rows=rows, want_cache=keep)
            if keep:
                prefix_cache[i] = c
        elif mode == "plain":
            pids = batch.tokens_of(pidx)
            P = len(pids)
            full_rows = None if rows is None else P + np.asarray(rows)
            if full_rows is None:
                full_rows = P + np.arange(len(ids))
            x, hid, _ = model.forward(np.concatenate([pids, ids]), capture_rows=full_rows)
            x = x[P:]
        else:
            if pidx not in prefix_cache:
                _, _, prefix_cache[pidx] = model.forward(batch.tokens_of(pidx), want_cache=True)
            c = prefix_cache[pidx]
            x, hid, _ = model.forward(ids, start_pos=c["len"], cache=c, capture_rows=rows)
        if i in capture:
            hidden[i] = np.stack(hid)
        for j in np.nonzero(batch.q_seq == i)[0]:
            p, f = model.decide(x[batch.q_marker[j]], int(batch.q_type[j]), batch.options_of(j))
            probs[int(j)] = p
            fields[int(j)] = f
    return {"probs": probs, "fields": fields, "hidden": hidden}
