"""CPU pins of the oracle's top-k select (the indexer's last step, upstream of
the decode's top-k list).

"Prime Inference: serving GLM-5.3 to agents is a KV-cache problem", section
"Decode: TP4, and the copies it keeps": an indexer picks the top cached
positions, at most 2,048 per query.  The logits themselves need the model's
weights and are not built; the select takes synthetic scores.

Pinned against: a closed form (scores that are a permutation of 0..L-1), the
rank definition checked by brute force on small inputs, the short-context
padding rule, and invariances under exact transforms of the scores.
"""
import numpy as np

import oracle


def test_permutation_scores_closed_form():
    rng = np.random.default_rng(1)
    L, K = 5000, 2048
    perm = rng.permutation(L)
    x = perm.astype(np.float32)[None]
    got = oracle.topk_select(x, np.array([L]), K)[0]
    # position i holds value perm[i]; the best K are the values L-1 .. L-K, in that order
    want = np.argsort(perm)[::-1][:K]
    assert np.array_equal(got, want)


def test_rank_definition_brute_force():
    rng = np.random.default_rng(2)
    for trial in range(300):
        L = int(rng.integers(0, 14))
        K = int(rng.integers(1, 10))
        x = rng.integers(-3, 4, size=(1, 16)).astype(np.float32)   # many ties
        got = oracle.topk_select(x, np.array([L]), K)[0]
        n = min(K, L)
        assert (got[n:] == -1).all()
        sel = got[:n]
        assert len(set(sel.tolist())) == n and all(0 <= i < L for i in sel)
        v = x[0, :L]
        for pos, i in enumerate(sel):
            # rank of i: entries strictly better, or equal and earlier
            better = sum(1 for j in range(L) if v[j] > v[i] or (v[j] == v[i] and j < i))
            assert better == pos, (trial, L, K, i)


def test_short_contexts_are_padded():
    x = np.arange(40, dtype=np.float32).reshape(2, 20)
    got = oracle.topk_select(x, np.array([3, 0]), 5)
    assert np.array_equal(got[0], [2, 1, 0, -1, -1])
    assert (got[1] == -1).all()
    # seq_lens beyond the row length are clamped to it
    got = oracle.topk_select(x, np.array([25, 20]), 21)
    assert np.array_equal(got[0, :20], np.arange(19, -1, -1)) and got[0, 20] == -1


def test_exact_transforms_keep_the_selection():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 3000)).astype(np.float32)
    lens = np.array([3000, 2500, 700])
    base = oracle.topk_select(x, lens, 512)
    assert np.array_equal(oracle.topk_select(x * np.float32(4.0), lens, 512), base)
    assert np.array_equal(oracle.topk_select(x * np.float32(0.5), lens, 512), base)
    # reversing a row reverses the positions (no ties in continuous data)
    rev = oracle.topk_select(x[:, ::-1].copy(), np.array([3000, 3000, 3000]), 512)
    full = oracle.topk_select(x, np.array([3000, 3000, 3000]), 512)
    assert np.array_equal(rev, 2999 - full)
