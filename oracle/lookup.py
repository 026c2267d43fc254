"""Reference of the prompt-lookup proposer and of verifying its proposals
(test infrastructure; only the tests and the benchmark's CPU leg use it).

The proposer ([QH] "Vấn đề 3: Làm sao khi không muốn train drafter?"): no
draft model; the candidates are the tokens that followed an earlier
occurrence of the text's current ending in the prompt or the output so far,
then the target verifies them.  The page leaves the details open; readings:

* the ending tried is the last n tokens, n from n_max down to n_min, the first
  n with an earlier occurrence wins;
* an earlier occurrence starts at i with i + n <= L - 1 (at least one token
  follows it inside the history); the earliest such i is taken;
* the candidates are the up to K tokens after it, clipped at the end of the
  history; no occurrence gives no candidates; a history length outside
  [0, Lmax] is invalid input (klen -1, which the verify step reports as an
  invalid sequence).

Verification ([MC] "Приёмка и почему распределение НЕ портится", [QH]
"Giải pháp"): a deterministic proposal is the draft distribution q that puts
all its mass on the proposed token (one-hot).  The acceptance rule then reads
accept x_j iff u_j < min(1, p_j(x_j) / 1) = p_j(x_j), and after a rejection the
residual max(0, p - q) is p with x_j removed.  A sequence with k_b candidates is
the verify step with K = k_b: after k_b acceptances the bonus token comes from
p_{k_b}.  Column K of the uniforms drives the final draw whatever k_b is.
Greedy sequences compare with the argmax as in the plain verify step.
"""

from __future__ import annotations

import numpy as np

from . import Result, verify_arrays


def propose(history: np.ndarray, hist_len: np.ndarray, n_max: int, n_min: int, K: int):
    """history [B, Lmax] int32 (row b holds hist_len[b] tokens) -> (cand [B, K]
    int32 padded with -1, klen [B] int32).  Plain loops, one sequence at a time."""
    if not (1 <= n_min <= n_max) or K < 0:
        raise ValueError("need 1 <= n_min <= n_max and K >= 0")
    B = history.shape[0]
    cand = np.full((B, K), -1, np.int32)
    klen = np.zeros(B, np.int32)
    for b in range(B):
        L = int(hist_len[b])
        if L < 0 or L > history.shape[1]:
            klen[b] = -1
            continue
        h = [int(t) for t in history[b, :L]]
        for n in range(min(n_max, L - 1), n_min - 1, -1):
            suffix = h[L - n:]
            found = -1
            for i in range(0, L - n):              # the continuation starts at i + n <= L - 1
                if h[i:i + n] == suffix:
                    found = i
                    break
            if found >= 0:
                c = found + n
                k = min(K, L - c)
                cand[b, :k] = h[c:c + k]
                klen[b] = k
                break
    return cand, klen


def onehot_rows(tokens: np.ndarray, V: int) -> np.ndarray:
    """Draft logits of a deterministic proposal: 0 at the proposed token, -inf
    elsewhere (every entry -inf for a token outside [0, V))."""
    k = tokens.shape[-1]
    d = np.full(tokens.shape[:-1] + (k, V), -np.inf, np.float64)
    for idx in np.ndindex(tokens.shape):
        t = int(tokens[idx])
        if 0 <= t < V:
            d[idx + (t,)] = 0.0
    return d


def verify_lookup(target, cand, klen, uniforms, T, greedy, B, K, V) -> Result:
    """The verify step on proposer candidates, one sequence at a time through
    the whole-step oracle with K = k_b and one-hot draft rows."""
    res = Result(
        accepted_len=np.full(B, -7, np.int32), out_tokens=np.full((B, K + 1), -1, np.int32),
        p_tok=np.full((B, K), np.nan), q_tok=np.full((B, K), np.nan),
        lse_p=np.full((B, K + 1), np.nan), lse_q=np.full((B, K), np.nan),
        res_mass=np.full(B, np.nan), test_margin=np.full((B, K), np.nan),
        draw_margin=np.full(B, np.nan), flags=np.zeros(B, np.int32))
    g_all = np.zeros(B, np.uint8) if greedy is None else np.asarray(greedy, np.uint8)
    for b in range(B):
        kb = int(klen[b])
        if kb < 0 or kb > K:
            res.accepted_len[b] = -1
            continue
        tgt = np.ascontiguousarray(target[b:b + 1, :kb + 1])
        tok = np.ascontiguousarray(cand[b:b + 1, :kb], np.int32)
        uni = np.concatenate([uniforms[b, :kb], uniforms[b, K:K + 1]])[None, :].astype(np.float32)
        g = g_all[b:b + 1]
        drf = onehot_rows(tok, V) if kb > 0 else None
        r = verify_arrays(tgt, drf, tok, uni, T, g, 1, kb, V, nthreads=1)
        res.accepted_len[b] = r.accepted_len[0]
        res.out_tokens[b, :kb + 1] = r.out_tokens[0]
        res.p_tok[b, :kb] = r.p_tok[0]
        res.q_tok[b, :kb] = r.q_tok[0]
        res.lse_p[b, :kb + 1] = r.lse_p[0]
        res.lse_q[b, :kb] = r.lse_q[0]
        res.res_mass[b] = r.res_mass[0]
        res.test_margin[b, :kb] = r.test_margin[0]
        res.draw_margin[b] = r.draw_margin[0]
        res.flags[b] = r.flags[0]
    return res
