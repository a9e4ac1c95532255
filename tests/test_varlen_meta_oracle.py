"""Pins of the oracle's sequence-aligned chunk table (pure integers).

The table is checked against a token-by-token brute force: every token of
sequence i belongs to chunk (i, (t - cu[i]) // C), chunks are numbered in
token order.  Exhaustive over all sequence-length patterns up to 4C for small
chunk sizes, plus random large cases.
"""
import itertools

import numpy as np

import oracle


def brute(cu, C):
    owner = []
    for i in range(len(cu) - 1):
        for t in range(cu[i], cu[i + 1]):
            owner.append((i, (t - cu[i]) // C, t))
    chunks = {}
    for i, k, t in owner:
        chunks.setdefault((i, k), []).append(t)
    keys = sorted(chunks)
    seq = [k[0] for k in keys]
    start = [chunks[k][0] for k in keys]
    length = [len(chunks[k]) for k in keys]
    first = [sum(1 for k in keys if k[0] < i) for i in range(len(cu))]
    return seq, start, length, first


def check(cu, C):
    m = oracle.varlen_chunk_meta(cu, C)
    seq, start, length, first = brute(cu, C)
    assert m.seq == seq and m.start == start and m.length == length
    assert m.first_chunk == first and m.nchunks == len(seq)
    T, nseq = cu[-1], len(cu) - 1
    assert m.nchunks <= -(-T // C) + nseq
    assert sum(m.length) == T
    assert all(1 <= L <= C for L in m.length)


def test_exhaustive_small():
    for C in (1, 2, 3, 4, 8):
        lens_range = range(0, 4 * C + 1)
        for nseq in (1, 2):
            for lens in itertools.product(lens_range, repeat=nseq):
                cu = [0] + list(np.cumsum(lens))
                check([int(v) for v in cu], C)


def test_three_sequences_around_edges():
    C = 4
    for lens in itertools.product([0, 1, 3, 4, 5, 8, 9], repeat=3):
        check([0] + [int(v) for v in np.cumsum(lens)], C)


def test_random_large():
    rng = np.random.default_rng(0)
    for _ in range(50):
        nseq = int(rng.integers(1, 40))
        T = int(rng.integers(nseq, 20000))
        cuts = np.sort(rng.choice(np.arange(0, T + 1), size=nseq - 1, replace=True))
        cu = [0] + [int(c) for c in cuts] + [T]
        check(cu, int(rng.choice([32, 64, 128, 256])))


def test_batch_meta_is_uniform_grid():
    m = oracle.batch_chunk_meta(3, 300, 128)
    assert m.nchunks == 9
    assert m.start == [0, 128, 256, 300, 428, 556, 600, 728, 856]
    assert m.length == [128, 128, 44] * 3
    assert m.first_chunk == [0, 3, 6, 9]
