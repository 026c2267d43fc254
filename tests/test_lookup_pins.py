"""CPU pins of the prompt-lookup oracle (oracle/lookup.py): the proposer
against worked examples and an independent substring search, and the one-hot
verification against the law the method guarantees."""

import numpy as np
import pytest

import oracle
from oracle import lookup


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _prop(seq, n_max, n_min, K):
    h = np.array([seq], np.int32)
    cand, klen = lookup.propose(h, np.array([len(seq)]), n_max, n_min, K)
    return cand[0, :klen[0]].tolist(), int(klen[0])


def test_propose_worked_examples():
    # the code-edit pattern of the page: the output re-types a span of the prompt
    # (tokens as small integers): prompt 10 11 12 13 14 15, output so far 11 12
    prompt = [10, 11, 12, 13, 14, 15]
    assert _prop(prompt + [11, 12], 3, 1, 3) == ([13, 14, 15], 3)
    # the continuation is clipped at the end of the history
    assert _prop(prompt + [13, 14], 2, 1, 8) == ([15, 13, 14], 3)
    # no earlier occurrence at any length: no candidates
    assert _prop(prompt + [99], 3, 1, 4) == ([], 0)
    # the longest ending wins: "12 13" occurs twice, "5 12 13" once
    assert _prop([12, 13, 7, 5, 12, 13, 8, 9, 5, 12, 13], 3, 1, 2) == ([8, 9], 2)
    # among equal lengths the earliest occurrence wins
    assert _prop([1, 2, 3, 1, 2, 4, 1, 2], 2, 1, 1) == ([3], 1)
    # an occurrence overlapping the ending itself (periodic text)
    assert _prop([7, 7, 7, 7], 2, 2, 5) == ([7, 7], 2)
    # n_min above every match length
    assert _prop([1, 2, 3, 1, 2], 3, 3, 4) == ([], 0)
    # histories too short to hold an earlier occurrence, and K = 0
    assert _prop([4], 2, 1, 3) == ([], 0)
    assert _prop([], 2, 1, 3) == ([], 0)
    assert _prop([1, 2, 1, 2], 2, 1, 0) == ([], 0)


def _by_string_search(seq, n_max, n_min, K):
    """The same rule through str.find on a letter encoding (an independent formulation)."""
    s = "".join(chr(97 + t) for t in seq)
    L = len(s)
    for n in range(n_max, n_min - 1, -1):
        if n > L - 1:
            continue
        i = s.find(s[L - n:])                    # earliest occurrence
        if i + n <= L - 1:                       # one that leaves a token after it
            c = i + n
            k = min(K, L - c)
            return list(seq[c:c + k]), k
    return [], 0


@pytest.mark.parametrize("alphabet", [2, 3, 5, 26])
def test_propose_matches_substring_search(alphabet):
    rng = np.random.default_rng(alphabet)
    for _ in range(400):
        L = int(rng.integers(0, 40))
        seq = rng.integers(0, alphabet, size=L).tolist()
        n_max = int(rng.integers(1, 6))
        n_min = int(rng.integers(1, n_max + 1))
        K = int(rng.integers(0, 7))
        assert _prop(seq, n_max, n_min, K) == _by_string_search(seq, n_max, n_min, K), (seq, n_max, n_min, K)


def test_propose_invalid_length():
    h = np.array([[1, 2, 1, 2], [1, 2, 1, 2], [1, 2, 1, 2]], np.int32)
    cand, klen = lookup.propose(h, np.array([-1, 5, 4]), 2, 1, 3)
    assert klen.tolist() == [-1, -1, 2] and np.all(cand[:2] == -1)


def test_propose_batched_rows_are_independent():
    rng = np.random.default_rng(5)
    B, Lmax = 9, 50
    h = rng.integers(0, 4, size=(B, Lmax)).astype(np.int32)
    ln = rng.integers(0, Lmax + 1, size=B)
    cand, klen = lookup.propose(h, ln, 4, 2, 5)
    for b in range(B):
        want = _by_string_search(h[b, :ln[b]].tolist(), 4, 2, 5)
        assert (cand[b, :klen[b]].tolist(), int(klen[b])) == want
        assert np.all(cand[b, klen[b]:] == -1)


def _dyadic_logits():
    # p = (1/2, 1/4, 1/8, 1/8) at T = 1
    return np.log(np.array([0.5, 0.25, 0.125, 0.125]))


def test_onehot_verify_reproduces_p_exactly():
    """With a one-hot proposal at x the first emitted token follows p_0 exactly:
    accept with probability p_0(x), else draw from p_0 without x.  Midpoint grids
    of u_0 and u_K (far from every boundary) give exact counts: N resolves the
    dyadic p_0(x), M = 2^4 * 3 * 7 the residuals (p without x, renormalised by
    1/2, 3/4 or 7/8)."""
    V, K = 4, 1
    l0 = _dyadic_logits()
    N, M = 64, 336
    for x in range(V):
        tgt = np.zeros((N * M, K + 1, V))
        tgt[:, 0, :] = l0
        tgt[:, 1, :] = l0
        cand = np.full((N * M, K), x, np.int32)
        klen = np.full(N * M, K, np.int32)
        u0 = (np.arange(N) + 0.5) / N
        uK = (np.arange(M) + 0.5) / M
        uni = np.stack([np.repeat(u0, M), np.tile(uK, N)], 1).astype(np.float32)
        r = lookup.verify_lookup(tgt, cand, klen, uni, 1.0, None, N * M, K, V)
        first = r.out_tokens[:, 0]
        counts = np.bincount(first, minlength=V)
        assert counts.tolist() == (np.exp(l0) * N * M).round().astype(int).tolist(), (x, counts)
        acc = r.accepted_len
        # accept iff u_0 < p_0(x)
        assert np.array_equal(acc == 1, uni[:, 0] < np.exp(l0[x]))
        # after a rejection the proposed token never comes back
        assert not np.any(first[acc == 0] == x)
        assert np.allclose(r.q_tok[:, 0], 1.0)


def test_onehot_verify_zero_candidates_is_a_plain_draw():
    rng = np.random.default_rng(3)
    B, K, V = 6, 3, 11
    tgt = rng.normal(size=(B, K + 1, V))
    uni = rng.random((B, K + 1)).astype(np.float32)
    r = lookup.verify_lookup(tgt, np.full((B, K), -1, np.int32), np.zeros(B, np.int32), uni, 0.9, None, B, K, V)
    assert np.all(r.accepted_len == 0)
    for b in range(B):
        p = np.exp((tgt[b, 0] - tgt[b, 0].max()) / 0.9)
        p /= p.sum()
        c = np.cumsum(p)
        assert r.out_tokens[b, 0] == int(np.searchsorted(c, float(uni[b, K]) * c[-1], side="right"))
        assert np.all(r.out_tokens[b, 1:] == -1)


def test_onehot_verify_ragged_lengths_and_bonus():
    """k_b candidates: after k_b acceptances the bonus token comes from p_{k_b}
    with u[b, K]; positions past k_b are never examined."""
    V, K = 5, 4
    l = np.full(V, -np.inf)
    l[2] = 0.0                                   # p = one-hot at token 2: every test of x = 2 passes
    tgt = np.tile(l, (3, K + 1, 1))
    tgt[:, 3, :] = np.log(np.array([0.1, 0.2, 0.3, 0.25, 0.15]))  # the bonus row of k_b = 3
    tgt[:, 4, 0] = np.nan                        # never examined
    cand = np.array([[2, 2, 2, 9], [2, 2, 2, 2], [2, 2, 2, 2]], np.int32)
    klen = np.array([3, 3, 5], np.int32)         # the last one is out of range: invalid
    uni = np.array([[0.9, 0.9, 0.9, 0.1, 0.05], [0.9, 0.9, 0.9, 0.1, 0.7], [0.5] * 5], np.float32)
    r = lookup.verify_lookup(tgt, cand, klen, uni, 1.0, None, 3, K, V)
    assert r.accepted_len.tolist() == [3, 3, -1]
    assert r.out_tokens[0].tolist() == [2, 2, 2, 0, -1]      # 0.05 < 0.1: token 0
    assert r.out_tokens[1].tolist() == [2, 2, 2, 3, -1]      # cumulative 0.6 <= 0.7 < 0.85: token 3
    assert r.out_tokens[2].tolist() == [-1] * (K + 1)


def test_onehot_verify_greedy_compares_with_argmax():
    V, K = 6, 3
    rng = np.random.default_rng(9)
    tgt = rng.normal(size=(2, K + 1, V))
    am = tgt.argmax(-1)
    cand = np.stack([am[0, :K], np.r_[am[1, 0], (am[1, 1] + 1) % V, am[1, 2]]]).astype(np.int32)
    r = lookup.verify_lookup(tgt, cand, np.array([3, 3], np.int32), np.zeros((2, K + 1), np.float32), 1.0,
                             np.ones(2, np.uint8), 2, K, V)
    assert r.accepted_len.tolist() == [3, 1]
    assert r.out_tokens[0].tolist() == am[0].tolist()
    assert r.out_tokens[1].tolist() == [am[1, 0], am[1, 1], -1, -1]
