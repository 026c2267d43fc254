"""CPU pins of the oracle side of the NEXT rows: the KV-cache commit and the
draft-side sampling step (the verify step with K = 0)."""

import numpy as np
import pytest

import oracle
from oracle import kvcache
from speculative_sampling_verification_06_amd import binding
from speculative_sampling_verification_06_amd import inputs as I


def encode(tok, pos):
    return np.array([tok, pos], np.int64).view(np.uint8)


def decode(row):
    t, p = np.asarray(row).view(np.int64)
    return int(t), int(p)


def test_commit_keeps_exactly_the_committed_stream():
    """Multi-round toy decode: every round the pass stages entries for the
    previous round's final token and the K candidates; after the commit the
    cache must hold exactly the committed tokens at their positions (the
    discarded suffix never becomes state)."""
    rng = np.random.default_rng(3)
    B, K, L, offset = 6, 4, 200, 1
    cache = np.zeros((1, B, L, 16), np.uint8)
    ln = np.zeros(B, np.int32)
    stream = [[] for _ in range(B)]
    pending = rng.integers(0, 1000, size=B)
    for _ in range(25):
        staged = np.zeros((1, B, K + offset, 16), np.uint8)
        cand = rng.integers(0, 1000, size=(B, K))
        for b in range(B):
            toks = [pending[b]] + list(cand[b])
            for i, t in enumerate(toks):
                staged[0, b, i] = encode(t, ln[b] + i)
        acc = rng.integers(-1, K + 1, size=B).astype(np.int32)
        cache, ln2, status = kvcache.kv_commit(cache, ln, staged, acc, offset)
        for b in range(B):
            if acc[b] < 0:
                assert status[b] == 1 and ln2[b] == ln[b]
                continue
            assert status[b] == 0
            stream[b] += [pending[b]] + list(cand[b, :acc[b]])
            pending[b] = rng.integers(0, 1000)
            assert ln2[b] == len(stream[b])
            for i, t in enumerate(stream[b]):
                assert decode(cache[0, b, i]) == (t, i)
            assert not cache[0, b, ln2[b]:].any() or ln2[b] == L, "nothing past the committed length"
        ln = ln2


def test_commit_refuses_overflow_and_leaves_state():
    cache = np.arange(2 * 3 * 5 * 4, dtype=np.uint8).reshape(2, 3, 5, 4)
    staged = np.full((2, 3, 3, 4), 7, np.uint8)
    ln = np.array([4, 1, 2], np.int32)
    acc = np.array([1, 2, -1], np.int32)
    new, ln2, st = kvcache.kv_commit(cache, ln, staged, acc, 1)
    assert list(st) == [2, 0, 1]
    assert list(ln2) == [4, 4, 2]
    assert np.array_equal(new[:, 0], cache[:, 0]) and np.array_equal(new[:, 2], cache[:, 2])
    assert np.all(new[:, 1, 1:4] == 7) and np.array_equal(new[:, 1, 4], cache[:, 1, 4])


def test_sampling_step_is_the_verify_step_without_tests():
    """K = 0: accepted_len 0 and the token is the inverse-CDF draw from p_0."""
    rng = np.random.default_rng(5)
    B, V, T = 64, 300, 0.7
    p = rng.dirichlet(np.ones(V) * 0.3, size=(B, 1))
    u = I.grid_uniforms(rng, (B, 1))
    w = I.from_probs(p, np.zeros((B, 0, V)), np.zeros((B, 0), np.int32), u, T=T)
    r = oracle.verify(w)
    assert np.all(r.accepted_len == 0)
    for b in range(B):
        cs = np.cumsum(p[b, 0])
        want = np.searchsorted(cs, float(u[b, 0]) * cs[-1], side="right")
        assert r.out_tokens[b, 0] == want or r.flags[b]


FAKE = 0x10000


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_sample_host_checks(lib):
    import ctypes as C
    assert lib.sv_sample(FAKE, 0, FAKE, C.c_float(1.0), None, -1, 10, FAKE, None, FAKE, 1 << 20, None) == -1
    assert lib.sv_sample(FAKE, 5, FAKE, C.c_float(1.0), None, 4, 10, FAKE, None, FAKE, 1 << 20, None) == -1
    assert lib.sv_sample(FAKE, 0, FAKE, C.c_float(0.0), None, 4, 10, FAKE, None, FAKE, 1 << 20, None) == -1
    assert lib.sv_sample(FAKE, 0, FAKE, C.c_float(1.0), None, 4, 10, FAKE, None, FAKE, 16, None) == -2
    assert lib.sv_sample(None, 0, None, C.c_float(1.0), None, 0, 10, None, None, None, 0, None) == 0
    assert binding.load_library().sv_sample_workspace_bytes(4, 10, 0) > binding.workspace_bytes(4, 0, 10, 0)


@pytest.mark.parametrize("kw", [dict(planes=0), dict(B=-1), dict(K=64), dict(offset=2), dict(l_max=0),
                                dict(row_bytes=0), dict(cache_len=None), dict(acc=None), dict(cache_len=FAKE + 2),
                                dict(status=FAKE + 1), dict(cache=None)])
def test_kv_commit_host_checks(lib, kw):
    a = dict(cache=FAKE, cache_len=FAKE, staged=FAKE, acc=FAKE, planes=2, B=3, K=4, offset=1, l_max=64,
             row_bytes=256, status=None)
    a.update(kw)
    assert lib.sv_kv_commit(a["cache"], a["cache_len"], a["staged"], a["acc"], a["planes"], a["B"], a["K"],
                            a["offset"], a["l_max"], a["row_bytes"], a["status"], None) == binding.SV_EINVAL


def test_kv_commit_empty_batch(lib):
    assert lib.sv_kv_commit(None, None, None, None, 1, 0, 4, 1, 10, 16, None, None) == 0


@pytest.mark.parametrize("kw", [dict(B=-1), dict(Lmax=-1), dict(n_min=0), dict(n_max=1, n_min=2), dict(n_max=65),
                                dict(K=-1), dict(K=64), dict(hist_len=None), dict(klen=None), dict(cand=None),
                                dict(history=None), dict(hist_len=FAKE + 2), dict(cand=FAKE + 1)])
def test_lookup_propose_host_checks(lib, kw):
    a = dict(history=FAKE, hist_len=FAKE, B=3, Lmax=50, n_max=4, n_min=1, K=5, cand=FAKE, klen=FAKE)
    a.update(kw)
    assert lib.sv_lookup_propose(a["history"], a["hist_len"], a["B"], a["Lmax"], a["n_max"], a["n_min"], a["K"],
                                 a["cand"], a["klen"], None) == -1


def test_lookup_propose_empty_batch(lib):
    assert lib.sv_lookup_propose(None, None, 0, 10, 4, 1, 5, None, None, None) == 0


def test_verify_lookup_host_checks(lib):
    import ctypes as C
    ws = 1 << 26
    args = lambda **kw: [kw.get("target", FAKE), kw.get("dt", 1), kw.get("cand", FAKE), kw.get("klen", FAKE), FAKE,
                         C.c_float(kw.get("T", 1.0)), None, kw.get("B", 4), kw.get("K", 3), kw.get("V", 100), FAKE,
                         FAKE, None, FAKE, kw.get("ws", ws), None]
    assert lib.spec_verify_lookup(*args(klen=None)) == -1
    assert lib.spec_verify_lookup(*args(klen=FAKE + 2)) == -1
    assert lib.spec_verify_lookup(*args(cand=None)) == -1
    assert lib.spec_verify_lookup(*args(dt=3)) == -1
    assert lib.spec_verify_lookup(*args(T=0.0)) == -1
    assert lib.spec_verify_lookup(*args(K=64)) == -1
    assert lib.spec_verify_lookup(*args(ws=16)) == -2
    assert lib.spec_verify_lookup(*args(B=0, klen=None)) == 0
