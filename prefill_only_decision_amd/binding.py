"""ctypes binding of libs1.so: argument marshalling only.

Every step of the path runs in the HIP library; this module converts Python
and numpy values into the C structs of include/s1.h and back.  PyTorch is
used by callers only for device buffers and stream handles (pass
`tensor.data_ptr()` and `stream.cuda_stream`).  Loading fails loudly when
the library has not been built.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libs1.so")

S1_OK, S1_EINVAL, S1_ENOMEM, S1_EDEVICE, S1_EBUDGET = 0, -1, -2, -3, -4
S1_F32, S1_BF16 = 0, 1
S1_CHOICE, S1_SCORE, S1_NOUL = 0, 1, 2
LORA_BITS = {"q": 1, "k": 2, "v": 4, "o": 8, "gate": 16, "up": 32, "down": 64}

# names declared in include/s1.h and include/s1_kernels.h
EXPORTS = (
    "s1_load_weights", "s1_prefill_decide", "s1_free", "s1_last_error", "s1_validate",
    "s1_plan_create", "s1_plan_run", "s1_plan_free", "s1_plan_tokens", "s1_plan_set_capture",
    "s1_plan_profile", "s1_plan_set_graph", "s1_plan_set_features", "s1_plan_set_invariant",
    "s1_plan_create_bucket", "s1_plan_update", "s1_plan_questions", "s1_plan_options",
    "s1_plan_set_layer_inputs",
    "s1k_gemm", "s1k_gemm_noalloc", "s1k_gemm_cfg", "s1k_gemm_resid_norm", "s1k_gemm_tile_configs", "s1k_frag_bytes", "s1k_frag_pack", "s1k_gemm_wfrag",
    "s1k_mfma_peak", "s1k_stream_copy", "s1k_stream_read",
    "s1k_rmsnorm", "s1k_embed", "s1k_lora_merge", "s1k_la_scan",
    "s1k_la_scan_chunked",
    "s1k_attention", "s1k_attention_plan", "s1k_readout", "s1k_vocab_lse", "s1k_token_logprobs", "s1k_gdn_scan",
)


class S1Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"s1 error {code}: {msg}")
        self.code = code


class Config(C.Structure):
    _fields_ = [
        ("n_layers", C.c_int32), ("full_every", C.c_int32),
        ("d_model", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
        ("la_heads", C.c_int32), ("la_dk", C.c_int32), ("la_dv", C.c_int32),
        ("fa_q_heads", C.c_int32), ("fa_kv_heads", C.c_int32), ("fa_head_dim", C.c_int32),
        ("rope_base", C.c_float), ("rms_eps", C.c_float),
        ("lora_rank", C.c_int32), ("lora_alpha", C.c_float), ("lora_targets", C.c_uint32),
        ("dtype", C.c_int32),
        ("max_tokens", C.c_int64), ("max_seqs", C.c_int32), ("max_questions", C.c_int32),
        ("max_options", C.c_int32), ("max_prefixes", C.c_int32), ("max_positions", C.c_int64),
        ("la_kind", C.c_int32),
    ]


class Tensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("dtype", C.c_int32), ("ndim", C.c_int32),
                ("shape", C.c_int64 * 2), ("data", C.c_void_p), ("on_device", C.c_int32)]


class Batch(C.Structure):
    _fields_ = [
        ("n_seqs", C.c_int32), ("cu_seqlens", C.POINTER(C.c_int32)),
        ("token_ids", C.POINTER(C.c_int32)), ("prefix_of", C.POINTER(C.c_int32)),
        ("n_questions", C.c_int32), ("q_seq", C.POINTER(C.c_int32)),
        ("q_marker", C.POINTER(C.c_int32)), ("q_type", C.POINTER(C.c_uint8)),
        ("opt_offsets", C.POINTER(C.c_int32)), ("opt_ids", C.POINTER(C.c_int32)),
    ]


class Decision(C.Structure):
    _fields_ = [("choice", C.c_int32), ("score", C.c_float), ("noul", C.c_float),
                ("answer_confidence", C.c_float), ("confidence", C.c_float),
                ("entropy_confidence", C.c_float)]


DECISION_DTYPE = np.dtype([("choice", np.int32), ("score", np.float32), ("noul", np.float32),
                           ("answer_confidence", np.float32), ("confidence", np.float32),
                           ("entropy_confidence", np.float32)])


class Features(C.Structure):
    _fields_ = [("n_targets", C.c_int32), ("rows", C.POINTER(C.c_int32)), ("tokens", C.POINTER(C.c_int32)),
                ("n_cands", C.c_int32), ("cand_offsets", C.POINTER(C.c_int32)),
                ("cand_group", C.POINTER(C.c_int32))]


class KernelTime(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_int32), ("total_us", C.c_double)]


class Timing(C.Structure):
    _fields_ = [("tokens_processed", C.c_int64), ("wall_us", C.c_double), ("device_us", C.c_double)]


_lib = None


def load_library(path=LIB_PATH):
    """Load libs1.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = C.CDLL(path)
    vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    sig = {
        "s1_load_weights": (C.c_int, [C.POINTER(Config), C.POINTER(Tensor), i32, vp, C.POINTER(vp)]),
        "s1_prefill_decide": (C.c_int, [vp, C.POINTER(Batch), vp, vp, C.POINTER(Timing), vp]),
        "s1_free": (None, [vp]),
        "s1_last_error": (C.c_char_p, []),
        "s1_validate": (C.c_int, [C.POINTER(Config), C.POINTER(Batch)]),
        "s1_plan_create": (C.c_int, [vp, C.POINTER(Batch), C.POINTER(vp)]),
        "s1_plan_run": (C.c_int, [vp, vp, vp, vp, vp]),
        "s1_plan_free": (None, [vp]),
        "s1_plan_tokens": (i64, [vp]),
        "s1_plan_set_capture": (C.c_int, [vp, i32, vp, vp]),
        "s1_plan_set_layer_inputs": (C.c_int, [vp, i32, vp, vp]),
        "s1_plan_set_graph": (C.c_int, [vp, i32]),
        "s1_plan_set_invariant": (C.c_int, [vp, i32]),
        "s1_plan_create_bucket": (C.c_int, [vp, i32, i32, i32, C.POINTER(vp)]),
        "s1_plan_update": (C.c_int, [vp, C.POINTER(Batch)]),
        "s1_plan_questions": (i32, [vp]),
        "s1_plan_options": (i64, [vp]),
        "s1_plan_set_features": (C.c_int, [vp, C.POINTER(Features), vp, vp, vp]),
        "s1_plan_profile": (C.c_int, [vp, vp, vp, vp, vp, C.POINTER(KernelTime), i32, C.POINTER(i32)]),
        "s1k_gemm": (C.c_int, [i32, vp, vp, vp, i32, i32, i32, i32, vp]),
        "s1k_gemm_cfg": (C.c_int, [i32, vp, vp, vp, i32, i32, i32, i32, i32, vp]),
        "s1k_gemm_noalloc": (C.c_int, [i32, vp, vp, vp, i32, i32, i32, i32, vp]),
        "s1k_gemm_resid_norm": (C.c_int, [vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp]),
        "s1k_gemm_tile_configs": (C.c_int, []),
        "s1k_frag_bytes": (i64, [i32, i32]),
        "s1k_mfma_peak": (C.c_int, [vp, i32, i32, vp, vp]),
        "s1k_stream_copy": (C.c_int, [vp, vp, i64, vp]),
        "s1k_stream_read": (C.c_int, [vp, i64, vp, vp]),
        "s1k_frag_pack": (C.c_int, [vp, i32, i32, i32, vp, vp]),
        "s1k_gemm_wfrag": (C.c_int, [vp, vp, vp, i32, i32, i32, i32, i32, vp]),
        "s1k_rmsnorm": (C.c_int, [i32, vp, vp, vp, i32, i32, f32, vp]),
        "s1k_embed": (C.c_int, [i32, vp, vp, vp, i32, i32, vp]),
        "s1k_lora_merge": (C.c_int, [i32, vp, vp, vp, vp, i32, i32, i32, f32, vp]),
        "s1k_la_scan": (C.c_int, [i32, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]),
        "s1k_la_scan_chunked": (C.c_int, [vp, vp, vp, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp]),
        "s1k_attention": (C.c_int, [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32, i32, vp]),
        "s1k_attention_plan": (C.c_int, [i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, i32,
                                         vp, vp]),
        "s1k_readout": (C.c_int, [i32, vp, i32, vp, f32, vp, i32, vp, vp, vp, vp, vp, vp, vp]),
        "s1k_vocab_lse": (C.c_int, [i32, vp, i32, vp, f32, vp, i32, i32, vp, vp, vp]),
        "s1k_gdn_scan": (C.c_int, [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]),
        "s1k_token_logprobs": (C.c_int, [i32, vp, i32, i32, vp, f32, vp, i32, i32, vp, vp, i32, vp, vp,
                                         vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(rc):
    if rc != S1_OK:
        raise S1Error(rc, load_library().s1_last_error().decode())
    return rc


def _ptr(a, ctype):
    return a.ctypes.data_as(C.POINTER(ctype)) if a is not None else None


def make_config(shape, max_tokens=None, max_seqs=64, max_questions=256, max_options=256,
                max_prefixes=4, max_positions=None):
    """s1_config from any object with the shape fields (n_layers, full_every,
    d_model, ffn, vocab, la_heads, la_dk, la_dv, fa_q_heads, fa_kv_heads,
    fa_head_dim, rope_base, rms_eps, lora_rank, lora_alpha, lora_targets,
    dtype "f32"/"bf16")."""
    c = Config()
    for f in ("n_layers", "full_every", "d_model", "ffn", "vocab", "la_heads", "la_dk", "la_dv",
              "fa_q_heads", "fa_kv_heads", "fa_head_dim", "lora_rank"):
        setattr(c, f, int(getattr(shape, f)))
    c.rope_base = float(shape.rope_base)
    c.rms_eps = float(shape.rms_eps)
    c.lora_alpha = float(shape.lora_alpha)
    c.lora_targets = sum(LORA_BITS[t] for t in shape.lora_targets)
    c.dtype = S1_BF16 if shape.dtype == "bf16" else S1_F32
    c.max_tokens = int(max_tokens or 8192)
    c.max_seqs = int(max_seqs)
    c.max_questions = int(max_questions)
    c.max_options = int(max_options)
    c.max_prefixes = int(max_prefixes)
    c.max_positions = int(max_positions or c.max_tokens)
    c.la_kind = 1 if getattr(shape, "la_kind", "gla") == "gdn" else 0
    return c


class _Arrays:
    """Keeps numpy arrays alive while a C struct points into them."""

    def __init__(self):
        self.keep = []

    def i32(self, a):
        a = np.ascontiguousarray(a, dtype=np.int32)
        self.keep.append(a)
        return a

    def u8(self, a):
        a = np.ascontiguousarray(a, dtype=np.uint8)
        self.keep.append(a)
        return a


def make_batch(b):
    """s1_batch from any object with cu_seqlens, token_ids, prefix_of, q_seq,
    q_marker, q_type, opt_offsets, opt_ids (numpy arrays)."""
    keep = _Arrays()
    cb = Batch()
    cu = keep.i32(b.cu_seqlens)
    cb.n_seqs = len(cu) - 1
    cb.cu_seqlens = _ptr(cu, C.c_int32)
    cb.token_ids = _ptr(keep.i32(b.token_ids), C.c_int32)
    cb.prefix_of = _ptr(keep.i32(b.prefix_of), C.c_int32) if b.prefix_of is not None else None
    qs = keep.i32(b.q_seq)
    cb.n_questions = len(qs)
    cb.q_seq = _ptr(qs, C.c_int32)
    cb.q_marker = _ptr(keep.i32(b.q_marker), C.c_int32)
    cb.q_type = _ptr(keep.u8(b.q_type), C.c_uint8)
    cb.opt_offsets = _ptr(keep.i32(b.opt_offsets), C.c_int32)
    cb.opt_ids = _ptr(keep.i32(b.opt_ids), C.c_int32)
    return cb, keep


def make_features(rows, tokens, cand_offsets=None, cand_group=None):
    """s1_features from target rows / tokens and candidate spans / groups."""
    keep = _Arrays()
    f = Features()
    r = keep.i32(rows)
    f.n_targets = len(r)
    f.rows = _ptr(r, C.c_int32)
    f.tokens = _ptr(keep.i32(tokens), C.c_int32)
    if cand_group is not None and len(cand_group):
        g = keep.i32(cand_group)
        f.n_cands = len(g)
        f.cand_offsets = _ptr(keep.i32(cand_offsets), C.c_int32)
        f.cand_group = _ptr(g, C.c_int32)
    else:
        f.n_cands = 0
    return f, keep


def validate(config, batch):
    """Host-only validation; returns the S1 status code (no exception)."""
    lib = load_library()
    cb, keep = make_batch(batch)
    return lib.s1_validate(C.byref(config), C.byref(cb))


def last_error():
    return load_library().s1_last_error().decode()


class Model:
    """A loaded model: owns the library handle until free()."""

    def __init__(self, config, tensors, stream=None):
        """tensors: dict name -> numpy array (host) or (device_ptr, shape)."""
        lib = load_library()
        self.config = config
        names, table = [], (Tensor * len(tensors))()
        self._keep = []
        for i, (name, t) in enumerate(tensors.items()):
            nb = name.encode()
            names.append(nb)
            e = table[i]
            e.name = nb
            e.dtype = config.dtype
            if isinstance(t, tuple):
                ptr, shape = t
                e.on_device = 1
                e.data = C.c_void_p(int(ptr))
            else:
                a = np.ascontiguousarray(t)
                self._keep.append(a)
                shape = a.shape
                e.on_device = 0
                e.data = a.ctypes.data_as(C.c_void_p)
            e.ndim = len(shape)
            e.shape[0] = int(shape[0])
            e.shape[1] = int(shape[1]) if len(shape) > 1 else 0
        self._names = names
        h = C.c_void_p()
        check(lib.s1_load_weights(C.byref(config), table, len(tensors), _stream(stream), C.byref(h)))
        self._keep = []
        self.handle = h

    def decide(self, batch, stream=None):
        """Host in, host out.  Returns (probs float32 [sum K], decisions
        structured array [Q], timing dict)."""
        lib = load_library()
        cb, keep = make_batch(batch)
        Q = cb.n_questions
        nopt = int(np.asarray(batch.opt_offsets)[-1]) if Q else 0
        probs = np.zeros(max(nopt, 1), np.float32)
        dec = np.zeros(max(Q, 1), DECISION_DTYPE)
        t = Timing()
        check(lib.s1_prefill_decide(self.handle, C.byref(cb), probs.ctypes.data_as(C.c_void_p),
                                    dec.ctypes.data_as(C.c_void_p), C.byref(t), _stream(stream)))
        return probs[:nopt], dec[:Q], {"tokens": t.tokens_processed, "wall_us": t.wall_us,
                                       "device_us": t.device_us}

    def plan(self, batch):
        return Plan(self, batch)

    def bucket_plan(self, max_tokens, max_questions, max_options):
        return Plan(self, bucket=(max_tokens, max_questions, max_options))

    def free(self):
        if self.handle:
            load_library().s1_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class Plan:
    """Resident-input plan of one request (token ids and metadata on device),
    or, with bucket=(max_tokens, max_questions, max_options), a length-bucket
    plan refilled by update()."""

    def __init__(self, model, batch=None, bucket=None):
        lib = load_library()
        self.model = model
        h = C.c_void_p()
        if bucket is not None:
            check(lib.s1_plan_create_bucket(model.handle, int(bucket[0]), int(bucket[1]), int(bucket[2]),
                                            C.byref(h)))
            self.handle = h
            self.n_questions = lib.s1_plan_questions(h)
            self.n_options = int(bucket[2]) + 2 * int(bucket[1])   # capacity of the outputs
        else:
            cb, keep = make_batch(batch)
            check(lib.s1_plan_create(model.handle, C.byref(cb), C.byref(h)))
            self.handle = h
            self.n_questions = cb.n_questions
            self.n_options = int(np.asarray(batch.opt_offsets)[-1]) if cb.n_questions else 0
        self.tokens = lib.s1_plan_tokens(h)

    def update(self, batch):
        """Refill a length-bucket plan with a one-sequence request."""
        cb, keep = make_batch(batch)
        check(load_library().s1_plan_update(self.handle, C.byref(cb)))

    def run(self, d_probs_ptr, d_dec_ptr, stream=None):
        """Enqueue the forward and readout; d_* are device pointers (ints)."""
        check(load_library().s1_plan_run(self.model.handle, self.handle, C.c_void_p(d_probs_ptr),
                                         C.c_void_p(d_dec_ptr), _stream(stream)))

    def profile(self, d_probs_ptr, d_dec_ptr, stream=None):
        """One synchronous run with per-launch events; returns
        {family: (launches, total_us)}."""
        out = (KernelTime * 32)()
        n = C.c_int32()
        check(load_library().s1_plan_profile(self.model.handle, self.handle, C.c_void_p(d_probs_ptr),
                                             C.c_void_p(d_dec_ptr), _stream(stream), out, 32, C.byref(n)))
        return {out[i].name.decode(): (out[i].launches, out[i].total_us) for i in range(n.value)}

    def set_graph(self, enable=True):
        check(load_library().s1_plan_set_graph(self.handle, 1 if enable else 0))

    def set_invariant(self, enable=True):
        check(load_library().s1_plan_set_invariant(self.handle, 1 if enable else 0))

    def set_capture(self, rows, d_hidden_ptr):
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        check(load_library().s1_plan_set_capture(self.handle, len(rows),
                                                 rows.ctypes.data_as(C.c_void_p),
                                                 C.c_void_p(d_hidden_ptr)))

    def set_layer_inputs(self, rows, d_src_ptr):
        """Before every layer l, replace the residual rows `rows` (packed
        token indices) by d_src[l, j, :] (fp32 device memory [n_layers,
        len(rows), d_model]); empty rows switch it off."""
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        check(load_library().s1_plan_set_layer_inputs(self.handle, len(rows),
                                                      rows.ctypes.data_as(C.c_void_p),
                                                      C.c_void_p(d_src_ptr)))

    def set_features(self, rows, tokens, cand_offsets, cand_group, d_logp_ptr, d_cand_logp_ptr=0,
                     d_cand_norm_ptr=0):
        """Full-vocabulary log-probabilities of (rows[n], tokens[n]) and the
        candidate scores, written by every following run; empty rows switch
        them off."""
        f, keep = make_features(rows, tokens, cand_offsets, cand_group)
        check(load_library().s1_plan_set_features(self.handle, C.byref(f), C.c_void_p(d_logp_ptr),
                                                  C.c_void_p(d_cand_logp_ptr or None),
                                                  C.c_void_p(d_cand_norm_ptr or None)))

    def free(self):
        if self.handle:
            load_library().s1_plan_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return C.c_void_p(s)
    return C.c_void_p(int(getattr(s, "cuda_stream", s)))


# ------------------------------------------------------------ kernel level
def _k(name, *args):
    return check(getattr(load_library(), name)(*[_arg(a) for a in args]))


def _arg(a):
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data_as(C.c_void_p)
    return a


def gemm(dtype, A, W, Cout, M, N, K, split_k=1, stream=None):
    return _k("s1k_gemm", dtype, C.c_void_p(A), C.c_void_p(W), C.c_void_p(Cout), M, N, K, split_k, _stream(stream))


def gemm_noalloc(dtype, A, W, Cout, M, N, K, split_k=1, stream=None):
    return _k("s1k_gemm_noalloc", dtype, C.c_void_p(A), C.c_void_p(W), C.c_void_p(Cout), M, N, K, split_k,
              _stream(stream))


def gemm_cfg(dtype, A, W, Cout, M, N, K, split_k, cfg, stream=None):
    return _k("s1k_gemm_cfg", dtype, C.c_void_p(A), C.c_void_p(W), C.c_void_p(Cout), M, N, K, split_k, cfg,
              _stream(stream))


def gemm_resid_norm(A, W, x, M, N, K, split_k, cfg, eps, hb, rs, stream=None):
    """Returns the form of hb: 1 = x * rs (a K split ran), 2 = x itself."""
    form = C.c_int32(0)
    _k("s1k_gemm_resid_norm", C.c_void_p(A), C.c_void_p(W), C.c_void_p(x), M, N, K, split_k, cfg,
       C.c_float(eps), C.c_void_p(hb), C.c_void_p(rs), C.byref(form), _stream(stream))
    return form.value


def gemm_tile_configs():
    return load_library().s1k_gemm_tile_configs()


def mfma_peak(seed, blocks, iters, out, stream=None):
    return _k("s1k_mfma_peak", C.c_void_p(seed), blocks, iters, C.c_void_p(out), _stream(stream))


def stream_copy(src, dst, nbytes, stream=None):
    return _k("s1k_stream_copy", C.c_void_p(src), C.c_void_p(dst), nbytes, _stream(stream))


def stream_read(src, nbytes, sink, stream=None):
    return _k("s1k_stream_read", C.c_void_p(src), nbytes, C.c_void_p(sink), _stream(stream))


def frag_bytes(N, K):
    return int(load_library().s1k_frag_bytes(N, K))


def frag_pack(W, N, K, gate_up16, out, stream=None):
    return _k("s1k_frag_pack", C.c_void_p(W), N, K, int(bool(gate_up16)), C.c_void_p(out), _stream(stream))


def gemm_wfrag(A, Wfrag, out, M, N, K, swiglu=False, tile=1, stream=None):
    return _k("s1k_gemm_wfrag", C.c_void_p(A), C.c_void_p(Wfrag), C.c_void_p(out), M, N, K, int(bool(swiglu)),
              tile, _stream(stream))


def rmsnorm(dtype, x, w, out, T, d, eps, stream=None):
    return _k("s1k_rmsnorm", dtype, C.c_void_p(x), C.c_void_p(w), C.c_void_p(out), T, d, C.c_float(eps), _stream(stream))


def embed(dtype, ids, E, x, T, d, stream=None):
    return _k("s1k_embed", dtype, C.c_void_p(ids), C.c_void_p(E), C.c_void_p(x), T, d, _stream(stream))


def lora_merge(dtype, W, A, B, out, out_dim, in_dim, rank, scale, stream=None):
    return _k("s1k_lora_merge", dtype, C.c_void_p(W), C.c_void_p(A) if A else None,
              C.c_void_p(B) if B else None, C.c_void_p(out), out_dim, in_dim, rank, C.c_float(scale),
              _stream(stream))


def la_scan(dtype, q, k, v, ld_qkv, log_g, o, T, H, dk, dv, cu_seqlens, s_init=None, s_final=None,
            stream=None):
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    return _k("s1k_la_scan", dtype, C.c_void_p(q), C.c_void_p(k), C.c_void_p(v), ld_qkv,
              C.c_void_p(log_g), C.c_void_p(o), T, H, dk, dv, len(cu) - 1, cu,
              C.c_void_p(s_init) if s_init else None, C.c_void_p(s_final) if s_final else None,
              _stream(stream))


def la_scan_chunked(q, k, v, ld_qkv, log_g, o, T, H, cu_seqlens, s_init=None, s_final=None, stream=None):
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    return _k("s1k_la_scan_chunked", C.c_void_p(q), C.c_void_p(k), C.c_void_p(v), ld_qkv, C.c_void_p(log_g),
              C.c_void_p(o), T, H, len(cu) - 1, cu, C.c_void_p(s_init) if s_init else None,
              C.c_void_p(s_final) if s_final else None, _stream(stream))


def attention(dtype, q, k, v, o, Hq, Hkv, hd, q_row0, q_len, kv_row0, kv_pre_row0, kv_pre_len,
              stream=None, block_rows=0, piece=0):
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (q_row0, q_len, kv_row0, kv_pre_row0, kv_pre_len)]
    return _k("s1k_attention", dtype, C.c_void_p(q), C.c_void_p(k), C.c_void_p(v), C.c_void_p(o),
              Hq, Hkv, hd, len(arrs[0]), *arrs, block_rows, piece, _stream(stream))


def attention_plan(q_row0, q_len, kv_row0, kv_pre_row0, kv_pre_len, Hq, block_rows=128, piece=-1, n_cu=256):
    """The attention launch plan on the host: (blocks int32 [n, 5] = (seq,
    q0, k_lo, k_hi, part), shared-prefix entries int32 [m, 5], row pieces
    from the smallest query row, chosen piece)."""
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (q_row0, q_len, kv_row0, kv_pre_row0, kv_pre_len)]
    n = len(arrs[0])
    rows = int(max([r + l for r, l in zip(arrs[0], arrs[1]) if l > 0], default=0)) + 1
    cap = 4096 + 64 * (rows + 1)
    blocks = np.zeros((cap, 5), np.int32)
    shared = np.zeros((max(n, 1), 5), np.int32)
    row_np = np.zeros(max(rows, 1), np.int32)
    nb, ns, pc = C.c_int32(), C.c_int32(), C.c_int32()
    _k("s1k_attention_plan", n, *arrs, Hq, block_rows, piece, n_cu, cap, blocks, C.byref(nb), len(shared), shared,
       C.byref(ns), len(row_np), row_np, C.byref(pc))
    return blocks[:nb.value].copy(), shared[:ns.value - n].copy(), row_np, pc.value


def readout(dtype, x, d, w_final, eps, E, Q, rows, opt_offsets, opt_ids, q_type, probs, decisions,
            stream=None):
    return _k("s1k_readout", dtype, C.c_void_p(x), d, C.c_void_p(w_final), C.c_float(eps), C.c_void_p(E), Q,
              C.c_void_p(rows), C.c_void_p(opt_offsets), C.c_void_p(opt_ids), C.c_void_p(q_type),
              C.c_void_p(probs), C.c_void_p(decisions), _stream(stream))


def vocab_lse(dtype, x, d, w_final, eps, E, V, R, rows, lse, stream=None):
    return _k("s1k_vocab_lse", dtype, C.c_void_p(x), d, C.c_void_p(w_final), C.c_float(eps), C.c_void_p(E), V, R,
              C.c_void_p(rows), C.c_void_p(lse), _stream(stream))


def token_logprobs(dtype, x, n_rows, d, w_final, eps, E, V, rows, tokens, cand_offsets, cand_group, logp,
                   cand_logp=0, cand_norm=0, stream=None):
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    g = np.ascontiguousarray(cand_group if cand_group is not None else [], dtype=np.int32)
    off = np.ascontiguousarray(cand_offsets if cand_offsets is not None else [0], dtype=np.int32)
    return _k("s1k_token_logprobs", dtype, C.c_void_p(x), n_rows, d, C.c_void_p(w_final), C.c_float(eps),
              C.c_void_p(E), V, len(rows), rows, tokens, len(g), off, g, C.c_void_p(logp),
              C.c_void_p(cand_logp or None), C.c_void_p(cand_norm or None), _stream(stream))


def gdn_scan(q, k, v, ld_qkv, log_g, beta, o, T, H, cu_seqlens, s_init=None, s_final=None, stream=None):
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    return _k("s1k_gdn_scan", C.c_void_p(q), C.c_void_p(k), C.c_void_p(v), ld_qkv, C.c_void_p(log_g),
              C.c_void_p(beta), C.c_void_p(o), T, H, len(cu) - 1, cu, C.c_void_p(s_init) if s_init else None,
              C.c_void_p(s_final) if s_final else None, _stream(stream))
