"""The split-key attention launch plan, checked on the host (no GPU): every
visible (query, key) pair is covered by exactly one workgroup, every row's
piece ordinals are 0 .. n-1 exactly once, pieces are cut at fixed key
positions (multiples of the piece), shared prefix sweeps serve only
sequences that continue that prefix, and the unsplit plan is one workgroup
per query block over its whole causal range; workgroups come heaviest
first."""
from collections import defaultdict

import numpy as np
import pytest

s1 = pytest.importorskip("prefill_only_decision_amd")


def _seqs(spec, shared_prefix=None):
    """spec: list of (q_len, prefix_len); rows packed in order; each prefix
    gets its own rows after the queries unless shared_prefix is set."""
    q_row0, q_len, kv_row0, pre_row0, pre_len = [], [], [], [], []
    r = 0
    for L, P in spec:
        q_row0.append(r); q_len.append(L); kv_row0.append(r); pre_len.append(P)
        r += L
    p = r
    for L, P in spec:
        pre_row0.append(r if shared_prefix else p)
        p += 0 if shared_prefix else P
    return q_row0, q_len, kv_row0, pre_row0, pre_len


def _check(seqs, bq, piece, n_cu=256):
    q_row0, q_len, kv_row0, pre_row0, pre_len = seqs
    blocks, shared, row_np, chosen = s1.binding.attention_plan(q_row0, q_len, kv_row0, pre_row0, pre_len, 16,
                                                                block_rows=bq, piece=piece, n_cu=n_cu)
    n = len(q_row0)
    live = [r for r, L in zip(q_row0, q_len) if L > 0]
    row_lo = min(live) if live else 0
    owner = {}
    for i in range(n):
        for t in range(q_len[i]):
            owner[q_row0[i] + t] = (i, t)
    cover = defaultdict(int)
    parts = defaultdict(list)
    for seq, q0, k_lo, k_hi, part in blocks:
        assert k_lo < k_hi
        if chosen > 0 and part >= 0 and k_hi - k_lo < chosen:
            # a piece never straddles a multiple of the piece size
            assert (k_lo // chosen) == ((k_hi - 1) // chosen)
        if seq < n:
            rows = [q_row0[seq] + t for t in range(q0, min(q0 + bq, q_len[seq]))]
            P = pre_len[seq]
        else:
            sr0, slen, _, spre_row0, sP = shared[seq - n]
            rows = [sr0 + t for t in range(q0, min(q0 + bq, slen))]
            P = sP
            assert k_hi <= sP
        for r in rows:
            i, t = owner[r]
            if seq >= n:   # a shared sweep serves sequences of that same prefix only
                assert pre_len[i] == P and pre_row0[i] == shared[seq - n][3]
            vis = [j for j in range(k_lo, k_hi) if j <= pre_len[i] + t]
            for j in vis:
                cover[(r, j)] += 1
            parts[r].append(part)
            if part < 0:
                assert k_lo == 0 and k_hi >= pre_len[i] + t + 1
    for r, (i, t) in owner.items():
        for j in range(pre_len[i] + t + 1):
            assert cover[(r, j)] == 1, (r, j, cover[(r, j)])
        ps = parts[r]
        if ps == [-1]:
            assert row_np[r - row_lo] == 1
        else:
            assert sorted(ps) == list(range(len(ps))) and row_np[r - row_lo] == len(ps), (r, ps)
    assert sum(cover.values()) == sum(pre_len[i] + t + 1 for r, (i, t) in owner.items())
    # workgroups are launched heaviest first: the 64-key blocks each sweeps
    # never increase along the plan
    def sweeps(b):
        seq, q0, k_lo, k_hi, _ = b
        if seq < n:
            L, P = q_len[seq], pre_len[seq]
        else:
            L, P = shared[seq - n][1], shared[seq - n][4]
        end = min(k_hi, P + min(q0 + bq, L))
        return -(-(end - k_lo) // 64) if end > k_lo else 0
    w = [sweeps(b) for b in blocks]
    assert all(a >= b for a, b in zip(w, w[1:])), w
    return blocks, shared, chosen


@pytest.mark.parametrize("spec", [
    [(1, 0), (100, 0), (128, 0), (129, 0), (300, 0), (512, 0)],
    [(64, 200), (1, 70), (130, 300), (0, 5)],
    [(512, 0)],
])
@pytest.mark.parametrize("piece", [0, 128, 192, 256, -1])
@pytest.mark.parametrize("bq", [32, 64, 128])
def test_plan_covers_every_visible_key_once(spec, piece, bq):
    if piece == 192:
        piece = 64 * 3
    _check(_seqs(spec), bq, piece)


@pytest.mark.parametrize("P,lens", [(2048, [64] * 6), (100, [64, 1, 65, 130]), (257, [3, 200]), (64, [1])])
@pytest.mark.parametrize("piece", [128, 1024, -1])
def test_shared_prefix_plan(P, lens, piece):
    blocks, shared, chosen = _check(_seqs([(L, P) for L in lens], shared_prefix=True), 128, piece)
    assert len(shared) == 1 and shared[0][1] == sum(lens) and shared[0][4] == P
    # the prefix keys are swept once per query block of the pooled queries
    n = len(lens)
    pre_blocks = [b for b in blocks if b[0] >= n]
    assert len(pre_blocks) == -(-sum(lens) // 128) * -(-P // chosen)


def test_unsplit_plan_is_one_workgroup_per_query_block():
    seqs = _seqs([(300, 0), (64, 200)])
    blocks, shared, chosen = _check(seqs, 128, 0)
    assert chosen == 0 and len(shared) == 0
    # heaviest first: 5, 5, 4 and 2 blocks of 64 keys, ties in plan order
    assert [tuple(b) for b in blocks] == [(0, 256, 0, 300, -1), (1, 0, 0, 264, -1), (0, 128, 0, 300, -1),
                                          (0, 0, 0, 300, -1)]


def test_auto_piece_fills_the_chip_for_one_short_request():
    # one 512-token request over 16 heads: unsplit, the longest chain is 8
    # blocks of 64 keys and only 64 workgroups run; the chosen piece bounds it
    blocks, _, chosen = _check(_seqs([(512, 0)]), 128, -1)
    assert chosen == 128 and len(blocks) * 16 >= 160
    # a long packed batch already fills the chip: no split
    spec = [(2048, 0)] * 8
    _, _, chosen = _check(_seqs(spec), 128, -1)
    assert chosen == 0
