"""Element-by-element comparison of the HIP path's outputs with the oracle's.

Test infrastructure (used by the GPU tests, the smoke check and the bench).

The bar:
* greedy sequences and invalid-input sequences: accepted length and every
  emitted token bit-exact;
* sampling sequences: accepted length and tokens identical, except where the
  oracle's own decision at the first point of divergence was within 1e-5 of
  its boundary:
  - lengths differ: the first position j = min(n_gpu, n_oracle) the two sides
    decided differently must have an oracle test margin |u_j - alpha_j| below
    1e-5 (a near test elsewhere in the sequence excuses nothing);
  - lengths agree: only the final token out[n] may differ, and only when the
    oracle flagged its final draw (u*S within 1e-5 of a CDF boundary, in
    probability units) or the draw fell back to p_n (residual mass 0);
  in both cases the GPU's row must still be a well-formed output: its
  accepted prefix equal to the draft tokens, a final token in [0, V), then -1
  padding.  Such sequences are counted as flagged mismatches;
* diagnostics where both examined the row: p(x), q(x) within 1e-5 relative
  (absolute floor 1e-30 for probabilities below fp32's normal range), the
  log-normalisers within 1e-5 relative (absolute floor 1e-5), the residual
  mass S within 1e-5 relative plus 2e-7 absolute (fp32 cancellation in
  p - q is absolute, about one ulp of the larger probability per token), NaN
  exactly where the oracle has NaN (rows neither side examined).
"""

from __future__ import annotations

import numpy as np

from . import FLAG_DRAW_NEAR, FLAG_FALLBACK, NEAR

P_RTOL, P_ATOL = 1e-5, 1e-30
LSE_RTOL, LSE_ATOL = 1e-5, 1e-5
S_RTOL, S_ATOL = 1e-5, 2e-7


class ParityError(AssertionError):
    pass


def _close(a, b, rtol, atol):
    return np.abs(a - b) <= atol + rtol * np.abs(b)


def _well_formed(row, n, tokens, V) -> bool:
    """An emitted row: x_0..x_{n-1} (the draft tokens), one token in [0, V), -1 after."""
    K1 = len(row)
    if not (0 <= n < K1):
        return False
    if not np.array_equal(row[:n], np.asarray(tokens[:n])):
        return False
    if not (0 <= int(row[n]) < V):
        return False
    return bool(np.all(row[n + 1:] == -1))


def compare(w, gpu: dict, orc, *, sequences=None, strict_diag=True) -> dict:
    """gpu: dict of numpy arrays (accepted_len, out_tokens and optional diagnostics).

    w supplies B, V, greedy and the draft tokens; sequences: the sequence
    indices that orc covers (default all, in order).  Returns a report;
    raises ParityError on any violation.
    """
    idx = np.arange(w.B) if sequences is None else np.asarray(sequences)
    g_acc = np.asarray(gpu["accepted_len"])[idx]
    g_out = np.asarray(gpu["out_tokens"])[idx]
    o_acc, o_out, flags = orc.accepted_len, orc.out_tokens, orc.flags
    margins = np.asarray(orc.test_margin)
    greedy = np.asarray(w.greedy)[idx] != 0
    tokens = np.asarray(w.tokens)
    tokens = tokens[idx] if tokens.ndim == 2 and tokens.shape[0] == w.B else tokens
    problems = []
    flagged_mismatch = []
    same_n = g_acc == o_acc
    for t, b in enumerate(idx):
        gn, on = int(g_acc[t]), int(o_acc[t])
        if gn == on and np.array_equal(g_out[t], o_out[t]):
            continue
        desc = f"gpu n={gn} {g_out[t].tolist()} vs oracle n={on} {o_out[t].tolist()}"
        if greedy[t] or on < 0 or gn < 0:
            problems.append(f"seq {b}: {desc} (greedy={bool(greedy[t])})")
            continue
        if not _well_formed(g_out[t], gn, tokens[t] if tokens.size else [], w.V):
            problems.append(f"seq {b}: malformed gpu row: {desc}")
            continue
        if gn != on:
            jd = min(gn, on)                       # first test decided differently
            mg = margins[t, jd] if margins.ndim == 2 and jd < margins.shape[1] else np.nan
            ok = bool(np.isfinite(mg) and mg < NEAR)
            why = f"test margin at position {jd} = {mg:.3g}"
        else:
            ok = bool(flags[t] & (FLAG_DRAW_NEAR | FLAG_FALLBACK))
            why = f"flags={int(flags[t])}"
        if ok:
            flagged_mismatch.append(int(b))
        else:
            problems.append(f"seq {b}: unflagged mismatch {desc} ({why})")

    diag_checked = 0
    if "p_tok" in gpu and strict_diag:
        ok_rows = same_n & (o_acc >= 0)
        for key, rtol, atol in (("p_tok", P_RTOL, P_ATOL), ("q_tok", P_RTOL, P_ATOL),
                                ("lse_p", LSE_RTOL, LSE_ATOL), ("lse_q", LSE_RTOL, LSE_ATOL)):
            g = np.asarray(gpu[key], np.float64)[idx][ok_rows]
            o = np.asarray(orc[key], np.float64)[ok_rows]
            if g.size == 0:
                continue
            nan_g, nan_o = np.isnan(g), np.isnan(o)
            if not np.array_equal(nan_g, nan_o):
                bad = np.argwhere(nan_g != nan_o)[:5]
                problems.append(f"{key}: NaN pattern differs at {bad.tolist()}")
            both = ~nan_g & ~nan_o
            cl = _close(g[both], o[both], rtol, atol)
            diag_checked += int(both.sum())
            if not np.all(cl):
                worst = np.max(np.abs(g[both] - o[both]) / np.maximum(np.abs(o[both]), 1e-300))
                problems.append(f"{key}: {int((~cl).sum())} entries outside tolerance, worst rel {worst:.3g}")
        g = np.asarray(gpu["res_mass"], np.float64)[idx]
        sel = ok_rows & ~greedy & np.isfinite(orc.res_mass) & ((flags & FLAG_FALLBACK) == 0)
        if sel.any():
            cl = _close(g[sel], orc.res_mass[sel], S_RTOL, S_ATOL)
            diag_checked += int(sel.sum())
            if not np.all(cl):
                problems.append(f"res_mass: {int((~cl).sum())} outside tolerance; "
                                f"gpu {g[sel][~cl][:3]} oracle {orc.res_mass[sel][~cl][:3]}")
        gsel = ok_rows & greedy
        if gsel.any() and not np.all(g[gsel] == 0.0):
            problems.append("res_mass of greedy sequences must be 0")

    report = dict(sequences=int(len(idx)), flagged=int(np.count_nonzero(flags)),
                  flagged_mismatch=flagged_mismatch, diag_checked=diag_checked,
                  invalid=int((o_acc < 0).sum()))
    if problems:
        raise ParityError("; ".join(problems[:12]) + (f" ... ({len(problems)} problems)" if len(problems) > 12 else ""))
    return report
