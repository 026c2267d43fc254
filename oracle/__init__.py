"""fp64 CPU oracle of the speculative-sampling verify step (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never does.  The C source in this directory shares no code with the
HIP library; both sides meet only at the seeded input generator.

* ``build()`` compiles ``spec_oracle.c`` with gcc into ``liboracle.so``.
* ``verify(w)`` runs the whole verify step on a :class:`Workload`.
* ``row_softmax``, ``row_argmax`` and ``draw`` expose the single steps so the
  tests can pin each one against closed forms.
* ``lmhead_logits`` is the fused-LM-head workload's target logits: the fp64
  product of the exact bf16 hidden states and weights (a library matmul used as
  one step, no rounding of the product).
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FLAG_TEST_NEAR, FLAG_DRAW_NEAR, FLAG_FALLBACK = 1, 2, 4
NEAR = 1e-5


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Diag(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("p_tok", "q_tok", "lse_p", "lse_q", "res_mass", "test_margin", "draw_margin", "flags")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = C.CDLL(_LIB)
        lib.oracle_row_softmax.restype = C.c_int
        lib.oracle_row_softmax.argtypes = [C.c_void_p, C.c_int, C.c_int32, C.c_double, C.c_void_p, C.c_void_p]
        lib.oracle_row_argmax.restype = C.c_int
        lib.oracle_row_argmax.argtypes = [C.c_void_p, C.c_int, C.c_int32, C.c_void_p]
        lib.oracle_draw.restype = C.c_int32
        lib.oracle_draw.argtypes = [C.c_void_p, C.c_int32, C.c_double, C.c_void_p, C.c_void_p]
        lib.oracle_verify.restype = C.c_int
        lib.oracle_verify.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_double,
                                      C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                      C.POINTER(_Diag), C.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError(f"unsupported logit storage {a.dtype}")


def row_softmax(row: np.ndarray, T: float = 1.0):
    """(valid, p[V], lse) for one stored row."""
    row = np.ascontiguousarray(row)
    p = np.empty(row.shape[-1], np.float64)
    lse = C.c_double(np.nan)
    ok = _load().oracle_row_softmax(_ptr(row), _dtype_code(row), row.shape[-1], float(T), _ptr(p), C.byref(lse))
    return bool(ok), p, lse.value


def row_argmax(row: np.ndarray):
    row = np.ascontiguousarray(row)
    idx = C.c_int32(-1)
    ok = _load().oracle_row_argmax(_ptr(row), _dtype_code(row), row.shape[-1], C.byref(idx))
    return bool(ok), idx.value


def draw(r: np.ndarray, u: float):
    """(y, S, margin) of the inverse-CDF draw from weights r with uniform u."""
    r = np.ascontiguousarray(r, np.float64)
    S = C.c_double(0.0)
    m = C.c_double(0.0)
    y = _load().oracle_draw(_ptr(r), r.shape[0], float(u), C.byref(S), C.byref(m))
    return int(y), S.value, m.value


class Result(dict):
    """accepted_len, out_tokens and diagnostics of one oracle call (numpy arrays)."""
    __getattr__ = dict.__getitem__


def verify_arrays(target, draft, tokens, uniforms, T, greedy, B, K, V, nthreads=None) -> Result:
    target = np.ascontiguousarray(target)
    dcode = _dtype_code(target)
    draft = None if draft is None else np.ascontiguousarray(draft)
    if draft is not None and draft.size == 0:
        draft = None
    ddcode = dcode if draft is None else _dtype_code(draft)
    tokens = np.ascontiguousarray(tokens, np.int32).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int32)
    uniforms = np.ascontiguousarray(uniforms, np.float32).reshape(B, K + 1)
    g = None if greedy is None else np.ascontiguousarray(greedy, np.uint8)
    acc = np.full(B, -7, np.int32)
    out = np.full((B, K + 1), -7, np.int32)
    res = Result(
        accepted_len=acc, out_tokens=out,
        p_tok=np.full((B, K), np.nan), q_tok=np.full((B, K), np.nan),
        lse_p=np.full((B, K + 1), np.nan), lse_q=np.full((B, K), np.nan),
        res_mass=np.full(B, np.nan), test_margin=np.full((B, K), np.nan),
        draw_margin=np.full(B, np.nan), flags=np.zeros(B, np.int32))
    dg = _Diag(*[_ptr(res[k]) for k in ("p_tok", "q_tok", "lse_p", "lse_q", "res_mass",
                                        "test_margin", "draw_margin", "flags")])
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    rc = _load().oracle_verify(_ptr(target), dcode, _ptr(draft), ddcode, _ptr(tokens) if K > 0 else None,
                               _ptr(uniforms), float(T), _ptr(g), B, K, V, _ptr(acc), _ptr(out),
                               C.byref(dg), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_verify rejected its arguments (rc={rc})")
    res["nthreads"] = min(int(nthreads), max(B, 1))
    return res


def verify(w, nthreads=None, target=None, sequences=None) -> Result:
    """Run the oracle on a Workload.  ``target`` overrides w.target (fused LM head);
    ``sequences`` restricts the call to a subset of sequence indices."""
    tgt = w.target if target is None else target
    drf, tok, uni, g = w.draft, w.tokens, w.uniforms, w.greedy
    B = w.B
    if sequences is not None:
        idx = np.asarray(sequences)
        tgt, drf, tok, uni, g = tgt[idx], drf[idx] if w.K > 0 else drf, tok[idx], uni[idx], g[idx]
        B = len(idx)
    return verify_arrays(tgt, drf if w.K > 0 else None, tok, uni, w.T, g, B, w.K, w.V, nthreads)


def lmhead_logits(hidden_bits: np.ndarray, w_bits: np.ndarray, rows=None, col_block: int = 8192) -> np.ndarray:
    """fp64 target logits = hidden @ W of the exact bf16 values, [B, K+1, V].

    ``rows`` (optional) selects sequence indices b; the result then has
    len(rows) sequences.  The product is a numpy float64 matmul.
    """
    def widen(b):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    h = hidden_bits if rows is None else hidden_bits[np.asarray(rows)]
    Bs, K1, d = h.shape
    V = w_bits.shape[1]
    h64 = widen(h.reshape(Bs * K1, d))
    out = np.empty((Bs * K1, V), np.float64)
    for c0 in range(0, V, col_block):
        out[:, c0:c0 + col_block] = h64 @ widen(w_bits[:, c0:c0 + col_block])
    return out.reshape(Bs, K1, V)


def time_verify(w, reps: int = 3, min_seconds: float = 0.0, nthreads=None):
    """Wall-clock the oracle on a workload: (median seconds per call, threads used, calls)."""
    ts = []
    t_start = time.perf_counter()
    res = None
    while len(ts) < reps or (time.perf_counter() - t_start) < min_seconds:
        t0 = time.perf_counter()
        res = verify(w, nthreads=nthreads)
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), res["nthreads"], len(ts)
