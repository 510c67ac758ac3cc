"""C-ABI contract on the CPU: the library loads without a GPU, exports every
function the headers declare, and rejects malformed requests with the right
error code before any device work (host-only validation)."""
import os
import re

import numpy as np
import pytest

from s1_workloads import make_batch, shape_of
from s1_workloads.batch import random_batch

s1 = pytest.importorskip("prefill_only_decision_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    try:
        return s1.load_library()
    except RuntimeError as e:
        pytest.fail(str(e))


def _declared():
    names = set()
    for h in ("s1.h", "s1_kernels.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"\b(s1k?_[a-z_]+)\s*\(", src):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert len(declared) >= 15
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, missing
    assert declared == set(s1.binding.EXPORTS)


def test_free_null_is_noop(lib):
    lib.s1_free(None)
    lib.s1_plan_free(None)


def test_gemm_config_count_and_validation(lib):
    n = s1.binding.gemm_tile_configs()
    assert n == 7
    # invalid configurations are rejected before any device work
    for cfg in (-1, n):
        with pytest.raises(s1.binding.S1Error) as e:
            s1.binding.gemm_cfg(s1.binding.S1_BF16, 16, 16, 16, 4, 4, 64, 1, cfg)
        assert e.value.code == -1   # S1_EINVAL


def test_frag_bytes_and_packed_gemm_validation(lib):
    # the fragment-order copy pads rows to whole 32-row blocks: 1 KB per
    # block and 16-column step
    assert s1.binding.frag_bytes(19456, 2560) == 19456 * 2560 * 2
    assert s1.binding.frag_bytes(6160, 2560) == 6176 * 2560 * 2
    assert s1.binding.frag_bytes(1, 16) == 32 * 16 * 2
    for n, k in ((0, 64), (64, 0), (64, 8), (64, 24)):
        assert s1.binding.frag_bytes(n, k) == 0
    # shapes the weight-direct GEMM does not take are rejected on the host
    bad = [dict(M=4, N=64, K=32), dict(M=4, N=64, K=100), dict(M=4, N=96, K=64, swiglu=True),
           dict(M=4, N=64, K=64, tile=0), dict(M=4, N=64, K=64, tile=5), dict(M=-1, N=64, K=64)]
    for kw in bad:
        with pytest.raises(s1.binding.S1Error) as e:
            s1.binding.gemm_wfrag(16, 16, 16, **kw)
        assert e.value.code == -1, kw
    with pytest.raises(s1.binding.S1Error):
        s1.binding.frag_pack(16, 96, 64, True, 16)     # gate/up packing needs N % 64 == 0
    for args in ((16, 0, 16), (16, 32, 8), (16, 32, -16)):   # null destination, ragged, negative
        with pytest.raises(s1.binding.S1Error) as e:
            s1.binding.stream_copy(*args)
        assert e.value.code == -1, args
    with pytest.raises(s1.binding.S1Error):
        s1.binding.mfma_peak(16, 0, 1, 16)


def _cfg(name="4b-single-512", **kw):
    return s1.make_config(shape_of(name), **kw)


def _mutate(b, **changes):
    import copy
    c = copy.deepcopy(b)
    for k, v in changes.items():
        setattr(c, k, v)
    return c


def _one_question(qtype, opts):
    from s1_workloads import Batch
    return Batch(cu_seqlens=np.array([0, 30], np.int32), token_ids=np.arange(30, dtype=np.int32),
                 prefix_of=np.array([-1], np.int32), q_seq=np.array([0], np.int32),
                 q_marker=np.array([29], np.int32), q_type=np.array([qtype], np.uint8),
                 opt_offsets=np.array([0, len(opts)], np.int32), opt_ids=np.array(opts, np.int32))


def test_valid_workloads_pass_validation():
    for name, kw in (("tiny-fp32", {}), ("4b-single-512", {}),
                     ("4b-varlen-16", dict(max_tokens=32768, max_positions=4096)),
                     ("4b-branch-4096x20", dict(max_tokens=8192)),
                     ("27b-single-1024", {})):
        assert s1.validate(_cfg(name, **kw), make_batch(name)) == s1.binding.S1_OK, s1.binding.last_error()


def test_empty_request_is_valid():
    b = random_batch(4096, [], seed=1)
    assert s1.validate(_cfg("tiny-fp32"), b) == 0


@pytest.mark.parametrize("case,code,needle", [
    ("k_lt_2", -1, "at least 2 options"),
    ("noul_k3", -1, "exactly 2 options"),
    ("marker_oob", -1, "marker outside"),
    ("bad_type", -1, "question type"),
    ("token_oob", -1, "token id out of range"),
    ("option_oob", -1, "option id out of range"),
    ("cu_decreasing", -1, "non-decreasing"),
    ("cu_start", -1, "cu_seqlens[0]"),
    ("too_many_tokens", -4, "max_tokens"),
    ("too_many_options", -4, "max_options"),
    ("prefix_chain", -1, "must not itself be a branch"),
    ("prefix_self", -1, "is invalid"),
    ("too_many_prefixes", -4, "max_prefixes"),
    ("q_seq_oob", -1, "q_seq out of range"),
    ("question_on_prefix", -1, "a question on a prefix sequence"),
])
def test_validation_errors(case, code, needle):
    cfg = _cfg("tiny-fp32", max_tokens=1024, max_options=16, max_prefixes=1)
    b = random_batch(4096, [30, 20, 10], seed=5, questions_per_seq=[2, 1, 1])
    if case == "k_lt_2":
        b.opt_offsets = b.opt_offsets.copy()
        b.opt_offsets[1:] = b.opt_offsets[1:] - (b.opt_offsets[1] - 1)
        b.opt_offsets[0] = 0
        b.opt_ids = b.opt_ids[-b.opt_offsets[-1]:] if b.opt_offsets[-1] > 0 else b.opt_ids
    elif case == "noul_k3":
        b = _one_question(2, [5, 6, 7])
    elif case == "marker_oob":
        b.q_marker = b.q_marker.copy()
        b.q_marker[0] = 30
    elif case == "bad_type":
        b.q_type = b.q_type.copy()
        b.q_type[0] = 3
    elif case == "token_oob":
        b.token_ids = b.token_ids.copy()
        b.token_ids[5] = 4096
    elif case == "option_oob":
        b.opt_ids = b.opt_ids.copy()
        b.opt_ids[0] = -1
    elif case == "cu_decreasing":
        b.cu_seqlens = np.array([0, 30, 20, 60], np.int32)
    elif case == "cu_start":
        b.cu_seqlens = b.cu_seqlens + 1
    elif case == "too_many_tokens":
        b = random_batch(4096, [1000, 100], seed=5)
    elif case == "too_many_options":
        b = _one_question(0, list(range(100, 120)))
    elif case == "prefix_chain":
        b.prefix_of = np.array([-1, 0, 1], np.int32)
    elif case == "prefix_self":
        b.prefix_of = np.array([-1, 1, -1], np.int32)
    elif case == "too_many_prefixes":
        b = random_batch(4096, [30, 20, 10, 5], seed=5, prefix_of=[-1, 0, -1, 2])
    elif case == "question_on_prefix":     # sequence 0 holds two questions
        b.prefix_of = np.array([-1, 0, -1], np.int32)
    elif case == "q_seq_oob":
        b.q_seq = b.q_seq.copy()
        b.q_seq[0] = 3
    rc = s1.validate(cfg, b)
    assert rc == code, (rc, s1.binding.last_error())
    assert needle in s1.binding.last_error()


def test_bad_config_rejected():
    cfg = _cfg("4b-single-512")
    cfg.la_dk = 64
    b = make_batch("4b-single-512")
    assert s1.validate(cfg, b) == -1
    assert "128" in s1.binding.last_error()


@pytest.mark.parametrize("kw,needle", [
    (dict(tokens=[0, 4096]), "token out of range"),
    (dict(rows=[0, 8]), "row out of range"),
    (dict(rows=[-1, 0]), "row out of range"),
    (dict(cand_offsets=[0, 2, 1], cand_group=[0, 0]), "decrease"),
    (dict(cand_offsets=[0, 1, 3], cand_group=[0, 0]), "exceed"),
    (dict(cand_offsets=[-1, 1], cand_group=[0]), "start"),
    (dict(d=102), "unsupported"),
    (dict(dtype=s1.binding.S1_BF16, d=256 + 64), "unsupported"),
])
def test_feature_request_validation(lib, kw, needle):
    """Malformed feature requests fail with S1_EINVAL on the host, before
    any device memory is touched (the pointers here are never dereferenced)."""
    a = dict(dtype=s1.binding.S1_F32, d=256, rows=[0, 7], tokens=[5, 9], cand_offsets=[0, 1, 2],
             cand_group=[3, 3])
    a.update(kw)
    with pytest.raises(s1.binding.S1Error) as e:
        s1.binding.token_logprobs(a["dtype"], 64, 8, a["d"], 64, 1e-6, 64, 4096, a["rows"], a["tokens"],
                                  a["cand_offsets"], a["cand_group"], 64, 64, 64)
    assert e.value.code == -1 and needle in str(e.value)
