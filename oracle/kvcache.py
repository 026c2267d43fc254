"""Reference of the KV-cache commit (test infrastructure).

After verification only the accepted prefix may become committed decoding
state (nalar.dev, "Speculative decoding: memverifikasi token draft secara
paralel", section "Verifikasi mengubah jalur cache").  This is the plain
definition of the staged-write commit, one sequence at a time.
"""

from __future__ import annotations

import numpy as np


def kv_commit(cache, cache_len, staged, accepted_len, offset):
    """cache [P, B, L, ...], cache_len [B], staged [P, B, S, ...] (or None for
    in-place entries), accepted_len [B]; returns (cache, cache_len, status) as
    new arrays.  c_b = accepted_len[b] + offset rows are committed."""
    cache = None if cache is None else np.array(cache, copy=True)
    ln = np.array(cache_len, dtype=np.int64, copy=True)
    acc = np.asarray(accepted_len)
    B = ln.shape[0]
    S = None if staged is None else staged.shape[2]
    L = None if cache is None else cache.shape[2]
    status = np.zeros(B, np.int32)
    for b in range(B):
        n = int(acc[b])
        if n < 0 or (S is not None and n > S - offset):
            status[b] = 1
            continue
        c = n + offset
        if ln[b] < 0 or (L is not None and ln[b] + c > L):
            status[b] = 2
            continue
        if staged is not None:
            cache[:, b, ln[b]:ln[b] + c] = staged[:, b, :c]
        ln[b] += c
    return cache, ln.astype(np.int32), status
