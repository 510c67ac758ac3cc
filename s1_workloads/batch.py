"""Seeded request batches: packed token ids, question markers, option ids."""
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .configs import WORKLOADS

QTYPE_CHOICE, QTYPE_SCORE, QTYPE_NOUL = 0, 1, 2


@dataclass
class Batch:
    """A packed batch of independent sequences (no padding).

    seq i occupies token rows cu_seqlens[i] .. cu_seqlens[i+1]-1.
    prefix_of[i] is -1, or the index of a question-free sequence whose tokens
    logically precede sequence i (a branch continues that prefix; branch token
    j sits at position len(prefix) + j).
    Question j reads the final hidden state of token q_marker[j] (0-based,
    within its own sequence) of sequence q_seq[j]; its options are
    opt_ids[opt_offsets[j]:opt_offsets[j+1]] in caller order (noul: [yes, no]).
    """
    cu_seqlens: np.ndarray      # int32 [n_seqs + 1]
    token_ids: np.ndarray       # int32 [T]
    prefix_of: np.ndarray       # int32 [n_seqs]
    q_seq: np.ndarray           # int32 [Q]
    q_marker: np.ndarray        # int32 [Q]
    q_type: np.ndarray          # uint8 [Q]
    opt_offsets: np.ndarray     # int32 [Q + 1]
    opt_ids: np.ndarray         # int32 [sum K]

    @property
    def n_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def n_questions(self) -> int:
        return len(self.q_seq)

    @property
    def seq_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def tokens_of(self, i: int) -> np.ndarray:
        return self.token_ids[self.cu_seqlens[i]:self.cu_seqlens[i + 1]]

    def options_of(self, j: int) -> np.ndarray:
        return self.opt_ids[self.opt_offsets[j]:self.opt_offsets[j + 1]]


def _assemble(seqs: List[np.ndarray], prefix_of: Sequence[int],
              questions: List[tuple]) -> Batch:
    """questions: list of (seq, marker, qtype, option_ids)."""
    lens = [len(s) for s in seqs]
    cu = np.zeros(len(seqs) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    toks = np.concatenate(seqs).astype(np.int32) if seqs else np.zeros(0, np.int32)
    offs = np.zeros(len(questions) + 1, np.int32)
    offs[1:] = np.cumsum([len(q[3]) for q in questions]) if questions else []
    opts = (np.concatenate([np.asarray(q[3], np.int32) for q in questions])
            if questions else np.zeros(0, np.int32))
    return Batch(
        cu_seqlens=cu, token_ids=toks,
        prefix_of=np.asarray(prefix_of, np.int32),
        q_seq=np.asarray([q[0] for q in questions], np.int32),
        q_marker=np.asarray([q[1] for q in questions], np.int32),
        q_type=np.asarray([q[2] for q in questions], np.uint8),
        opt_offsets=offs, opt_ids=opts.astype(np.int32))


def _opts(rng, vocab: int, k: int) -> np.ndarray:
    return rng.choice(vocab, size=k, replace=False).astype(np.int32)


def _k_for(rng, qtype: int, choice_range=(2, 8), score_k=5) -> int:
    if qtype == QTYPE_NOUL:
        return 2
    if qtype == QTYPE_SCORE:
        return score_k
    return int(rng.integers(choice_range[0], choice_range[1] + 1))


def random_batch(vocab: int, seq_lens: Sequence[int], seed,
                 questions_per_seq: Optional[Sequence[int]] = None,
                 prefix_of: Optional[Sequence[int]] = None,
                 choice_range=(2, 8), score_k=5) -> Batch:
    """Generic seeded batch for tests: uniform token ids; per sequence the
    given number of questions (default 1..3) with distinct markers, the last
    one on the final token; types uniform; options distinct ids."""
    tok_rng = np.random.default_rng([int(s) for s in np.atleast_1d(seed)] + [1])
    lay_rng = np.random.default_rng([int(s) for s in np.atleast_1d(seed)] + [2])
    n = len(seq_lens)
    prefix_of = list(prefix_of) if prefix_of is not None else [-1] * n
    is_prefix = {p for p in prefix_of if p >= 0}
    seqs = [tok_rng.integers(0, vocab, L).astype(np.int32) for L in seq_lens]
    qs = []
    for i, L in enumerate(seq_lens):
        if i in is_prefix or L == 0:
            continue
        nq = (questions_per_seq[i] if questions_per_seq is not None
              else int(lay_rng.integers(1, 4)))
        nq = min(nq, L)
        if nq <= 0:
            continue
        marks = sorted(lay_rng.choice(L - 1, size=nq - 1, replace=False).tolist()) \
            if nq > 1 else []
        marks.append(L - 1)
        for m in marks:
            t = int(lay_rng.integers(0, 3))
            qs.append((i, m, t, _opts(lay_rng, vocab, _k_for(lay_rng, t, choice_range, score_k))))
    return _assemble(seqs, prefix_of, qs)


def make_batch(name: str) -> Batch:
    """The batch of a named workload (see s1_workloads.configs.WORKLOADS)."""
    w = WORKLOADS[name]
    V = w.shape.vocab
    tok_rng = np.random.default_rng([w.workload_id, 1])
    lay_rng = np.random.default_rng([w.workload_id, 2])
    if name in ("tiny-fp32", "4b-single-512", "4b-gdn-single-512"):
        L = 128 if name == "tiny-fp32" else 512
        seqs = [tok_rng.integers(0, V, L).astype(np.int32)]
        marks = [63, 95, 127] if L == 128 else [383, 447, 511]
        spec = [(QTYPE_CHOICE, 3), (QTYPE_SCORE, 4), (QTYPE_NOUL, 2)]
        qs = [(0, m, t, _opts(lay_rng, V, k)) for m, (t, k) in zip(marks, spec)]
        return _assemble(seqs, [-1], qs)
    if name == "4b-varlen-16":
        lens = lay_rng.integers(256, 2049, 16)
        seqs = [tok_rng.integers(0, V, int(L)).astype(np.int32) for L in lens]
        qs = []
        for i, L in enumerate(lens):
            L = int(L)
            nq = int(lay_rng.integers(1, 7))
            marks = sorted(lay_rng.choice(L - 1, size=nq - 1, replace=False).tolist())
            marks.append(L - 1)
            for m in marks:
                t = int(lay_rng.integers(0, 3))
                qs.append((i, m, t, _opts(lay_rng, V, _k_for(lay_rng, t, (2, 8), 5))))
        return _assemble(seqs, [-1] * 16, qs)
    if name == "4b-branch-4096x20":
        seqs = [tok_rng.integers(0, V, 4096).astype(np.int32)]
        seqs += [tok_rng.integers(0, V, 64).astype(np.int32) for _ in range(20)]
        types = [QTYPE_CHOICE] * 8 + [QTYPE_SCORE] * 8 + [QTYPE_NOUL] * 4
        qs = []
        for j, t in enumerate(types):
            qs.append((j + 1, 63, t, _opts(lay_rng, V, _k_for(lay_rng, t, (3, 10), 5))))
        return _assemble(seqs, [-1] + [0] * 20, qs)
    if name == "27b-single-1024":
        seqs = [tok_rng.integers(0, V, 1024).astype(np.int32)]
        qs = [(0, 1023, QTYPE_CHOICE, _opts(lay_rng, V, 10))]
        return _assemble(seqs, [-1], qs)
    raise KeyError(name)
