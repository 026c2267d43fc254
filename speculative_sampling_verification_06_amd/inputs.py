"""Seeded synthetic inputs for the speculative-sampling verify step.

This module is shared by the tests, the benchmark and the smoke check, and is
the only code that both the HIP path and the fp64 oracle consume.  It holds none
of the verify step's arithmetic: no softmax normaliser, no acceptance ratio, no
residual and no inverse-CDF draw.  It only draws numbers:

* target logits  l ~ N(0, sigma) (+ an optional log-Zipf bias over token index),
* draft logits   d = a * l + N(0, sigma_d)   (the draft model's stand-in),
* draft tokens   x_j ~ softmax(d_j / T), drawn by the Gumbel-max construction
                 (argmax of d/T + Gumbel noise), or argmax d_j for greedy rows,
* uniforms       u on the 2^-24 grid in [0, 1),
* bf16 values    by round-to-nearest-even of the fp32 value, done once here so
                 that both sides read identical bits.

The workloads are the five synthetic configurations named for this method
(tiny, 32k-vocab fp32, 128k-vocab bf16 half greedy, 152k-vocab bf16, fused
LM head).  N(mu, sigma) takes sigma as the standard deviation.  The Zipf bias
is z_i = -1.1 * ln(i + 1), so softmax(z) alone is the Zipf(1.1) law over the
token index.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32, BF16, F64 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", F64: "f64"}

_WORKERS = 8


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def logits_as_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float64 view of stored logits (fp32, bf16 bits or fp64)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def zipf_bias(V: int, s: float = 1.1) -> np.ndarray:
    return (-s * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)


def grid_uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms on the 2^-24 grid in [0, 1), exactly representable in fp32."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def gumbel_argmax(rng: np.random.Generator, scores: np.ndarray) -> np.ndarray:
    """argmax over the last axis of scores + Gumbel(0,1) noise (Gumbel-max draw)."""
    u = rng.random(scores.shape)            # [0, 1)
    u = np.maximum(u, 1e-300)
    g = -np.log(-np.log(u))
    return np.argmax(scores + g, axis=-1).astype(np.int32)


@dataclasses.dataclass
class Workload:
    """One verify call's inputs, host side (numpy)."""
    name: str
    B: int
    K: int
    V: int
    dtype: int                 # F32 / BF16 / F64 (f64 only for oracle-only tests)
    T: float
    target: np.ndarray         # [B, K+1, V]  float32, uint16 (bf16 bits) or float64
    draft: np.ndarray          # [B, K, V]    same storage dtype
    tokens: np.ndarray         # [B, K] int32
    uniforms: np.ndarray       # [B, K+1] float32 in [0, 1)
    greedy: np.ndarray         # [B] uint8
    seed: int = 0
    hidden: np.ndarray | None = None   # fused LM-head workload: [B, K+1, d] bf16 bits
    w_lm: np.ndarray | None = None     # fused LM-head workload: [d, V] bf16 bits

    @property
    def verified_logits(self) -> int:
        return self.B * (self.K + 1) * self.V

    @property
    def elem_bytes(self) -> int:
        return {F32: 4, BF16: 2, F64: 8}[self.dtype]


def _store(x32: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    if dtype == F64:
        return x32.astype(np.float64)
    return np.ascontiguousarray(x32, dtype=np.float32)


def _stored_as_f64(x: np.ndarray, dtype: int) -> np.ndarray:
    return logits_as_f64(x, dtype)


def _seq_seeds(seed: int, B: int, nstream: int):
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(B)
    return [k.spawn(nstream) for k in kids]


def synth_logits(seed: int, B: int, K: int, V: int, *, dtype: int, T: float,
                 sigma: float, zipf: bool, draft_scale: float, draft_sigma: float,
                 greedy_mask: np.ndarray | None = None, name: str = "custom",
                 draft_from_target_rows: bool = True) -> Workload:
    """Generic recipe: l = N(0, sigma) [+ zipf]; d = draft_scale * l[:, :K] + N(0, draft_sigma).

    Draft tokens: Gumbel-max draw from softmax(d/T) for sampling sequences,
    argmax d for greedy sequences.  One independent PCG64 stream per sequence
    and purpose (logits, draft noise, tokens, uniforms), so the result does not
    depend on the thread count.
    """
    target = np.empty((B, K + 1, V), dtype={F32: np.float32, BF16: np.uint16, F64: np.float64}[dtype])
    draft = np.empty((B, K, V), dtype=target.dtype)
    tokens = np.empty((B, K), dtype=np.int32)
    uniforms = np.empty((B, K + 1), dtype=np.float32)
    greedy = np.zeros(B, dtype=np.uint8) if greedy_mask is None else greedy_mask.astype(np.uint8)
    bias = zipf_bias(V) if zipf else None
    seeds = _seq_seeds(seed, B, 4)

    def one(b):
        r_l, r_d, r_x, r_u = (np.random.Generator(np.random.PCG64(s)) for s in seeds[b])
        l = r_l.standard_normal((K + 1, V), dtype=np.float32) * np.float32(sigma)
        if bias is not None:
            l += bias
        d = (np.float32(draft_scale) * l[:K] +
             r_d.standard_normal((K, V), dtype=np.float32) * np.float32(draft_sigma))
        target[b] = _store(l, dtype)
        draft[b] = _store(d, dtype)
        dq = _stored_as_f64(draft[b], dtype)       # the values the verify step will read
        if K > 0:
            if greedy[b]:
                tokens[b] = np.argmax(dq, axis=-1).astype(np.int32)
            else:
                tokens[b] = gumbel_argmax(r_x, dq / T)
        uniforms[b] = grid_uniforms(r_u, (K + 1,))

    with ThreadPoolExecutor(max_workers=min(_WORKERS, max(1, B))) as ex:
        list(ex.map(one, range(B)))
    return Workload(name=name, B=B, K=K, V=V, dtype=dtype, T=T, target=target, draft=draft,
                    tokens=tokens, uniforms=uniforms, greedy=greedy, seed=seed)


# ---------------------------------------------------------------------------
# The five named workloads.  Seed = 1000 + index unless overridden.
# ---------------------------------------------------------------------------

def tiny(seed: int = 1000, greedy: bool = False) -> Workload:
    """B=1, K=4, V=32 fp32; l ~ N(0,2) iid; d = l + N(0,1); T=1."""
    return synth_logits(seed, 1, 4, 32, dtype=F32, T=1.0, sigma=2.0, zipf=False,
                        draft_scale=1.0, draft_sigma=1.0,
                        greedy_mask=np.array([1 if greedy else 0]),
                        name="tiny_greedy" if greedy else "tiny")


def cfg_32k(seed: int = 1001) -> Workload:
    """B=8, K=4, V=32000 fp32; l = N(0,3) + zipf; d = l + N(0,0.5); T=1, sampling."""
    return synth_logits(seed, 8, 4, 32000, dtype=F32, T=1.0, sigma=3.0, zipf=True,
                        draft_scale=1.0, draft_sigma=0.5, name="B8_K4_V32000_f32")


def cfg_128k(seed: int = 1002, B: int = 64) -> Workload:
    """B=64, K=5, V=128256 bf16; l = N(0,3) + zipf; d = 0.7 l + N(0,1.5); T=0.7; even b greedy."""
    mask = (np.arange(B) % 2 == 0).astype(np.uint8)
    return synth_logits(seed, B, 5, 128256, dtype=BF16, T=0.7, sigma=3.0, zipf=True,
                        draft_scale=0.7, draft_sigma=1.5, greedy_mask=mask,
                        name="B64_K5_V128256_bf16_halfgreedy")


def cfg_152k(seed: int = 1003, B: int = 256) -> Workload:
    """B=256, K=8, V=152064 bf16; l = N(0,4) + zipf; d = l + N(0,2.5); T=1, sampling."""
    return synth_logits(seed, B, 8, 152064, dtype=BF16, T=1.0, sigma=4.0, zipf=True,
                        draft_scale=1.0, draft_sigma=2.5, name=f"B{B}_K8_V152064_bf16")


def cfg_vocab_shard(seed: int = 1003, B: int = 256, shards: int = 8) -> Workload:
    """One GPU's share of the B=256, K=8, V=152064 workload when the LM head is
    split over the vocabulary: the first V/shards = 19008 columns (the head of
    the Zipf bias), same recipe otherwise."""
    V = 152064 // shards
    return synth_logits(seed, B, 8, V, dtype=BF16, T=1.0, sigma=4.0, zipf=True,
                        draft_scale=1.0, draft_sigma=2.5, name=f"B{B}_K8_V{V}_bf16_vocab_shard")


def cfg_lmhead(seed: int = 1004, B: int = 32, K: int = 5, d: int = 4096, V: int = 128256,
               draft_noise: float = 1.0, T: float = 0.8) -> Workload:
    """Fused LM head: hidden bf16 [B,K+1,d] ~ N(0,1); W bf16 [d,V] ~ N(0,0.02).

    The draft logits stand in for a draft model that tracks the target: they are
    (hidden @ W)[:, :K] + N(0,1), rounded to bf16.  The product here is a plain
    fp32 numpy matmul used only to synthesise that stand-in; the verify step's
    own target logits come from the HIP GEMM (and, for checking, from the
    oracle's fp64 product).
    """
    ss = np.random.SeedSequence(seed)
    r_h, r_w, r_d, r_x, r_u = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5))
    hidden = f32_to_bf16_bits(r_h.standard_normal((B, K + 1, d), dtype=np.float32))
    w = f32_to_bf16_bits(r_w.standard_normal((d, V), dtype=np.float32) * np.float32(0.02))
    h32 = bf16_bits_to_f32(hidden[:, :K, :]).reshape(B * K, d)
    base = np.empty((B * K, V), dtype=np.float32)
    step = 16384
    for c0 in range(0, V, step):
        base[:, c0:c0 + step] = h32 @ bf16_bits_to_f32(w[:, c0:c0 + step])
    dl = base.reshape(B, K, V) + r_d.standard_normal((B, K, V), dtype=np.float32) * np.float32(draft_noise)
    draft = f32_to_bf16_bits(dl)
    dq = bf16_bits_to_f32(draft).astype(np.float64)
    tokens = np.empty((B, K), dtype=np.int32)
    for b in range(B):
        tokens[b] = gumbel_argmax(r_x, dq[b] / T)
    uniforms = grid_uniforms(r_u, (B, K + 1))
    return Workload(name=f"lmhead_B{B}_K{K}_d{d}_V{V}_bf16", B=B, K=K, V=V, dtype=BF16, T=T,
                    target=np.empty((0,), np.uint16), draft=draft, tokens=tokens,
                    uniforms=uniforms, greedy=np.zeros(B, np.uint8), seed=seed,
                    hidden=hidden, w_lm=w)


CONFIGS = {
    "tiny": tiny,
    "tiny_greedy": lambda seed=1000: tiny(seed, greedy=True),
    "cfg32k": cfg_32k,
    "cfg128k": cfg_128k,
    "cfg152k": cfg_152k,
    "lmhead": cfg_lmhead,
    # one GPU's share of cfg152k over 8 GPUs: by batch, or by vocabulary
    "shard_batch": lambda seed=1003: cfg_152k(seed, B=32),
    "shard_vocab": cfg_vocab_shard,
}


def from_probs(p: np.ndarray, q: np.ndarray, tokens: np.ndarray, uniforms: np.ndarray,
               T: float = 1.0, dtype: int = F64, greedy: np.ndarray | None = None,
               name: str = "from_probs") -> Workload:
    """Build a workload whose softmax(l/T) and softmax(d/T) are the given laws.

    Logits are T * ln(prob) (ln 0 = -inf).  Used by tests that state the
    distributions directly (the worked example, closed forms, enumeration).
    p: [B, K+1, V]; q: [B, K, V].
    """
    with np.errstate(divide="ignore"):
        lt = T * np.log(np.asarray(p, np.float64))
        ld = T * np.log(np.asarray(q, np.float64))
    B, K1, V = lt.shape
    if dtype == F64:
        tgt, dft = lt, ld
    elif dtype == F32:
        tgt, dft = lt.astype(np.float32), ld.astype(np.float32)
    else:
        tgt, dft = f32_to_bf16_bits(lt.astype(np.float32)), f32_to_bf16_bits(ld.astype(np.float32))
    g = np.zeros(B, np.uint8) if greedy is None else np.asarray(greedy, np.uint8)
    return Workload(name=name, B=B, K=K1 - 1, V=V, dtype=dtype, T=T,
                    target=np.ascontiguousarray(tgt), draft=np.ascontiguousarray(dft),
                    tokens=np.ascontiguousarray(tokens, np.int32),
                    uniforms=np.ascontiguousarray(uniforms, np.float32), greedy=g)


def eager_bytes(w: Workload) -> int:
    """Bytes of logits one eager verify reads once: every target row, and draft rows of sampling sequences."""
    s = w.elem_bytes
    n_samp = int((w.greedy == 0).sum())
    return w.B * (w.K + 1) * w.V * s + n_samp * w.K * w.V * s


def needed_bytes(w: Workload, accepted_len: np.ndarray) -> int:
    """Bytes the method itself needs, given each sequence's accepted length n.

    Rows past the first rejection are never examined: (n+1) target rows, plus
    min(n+1, K) draft rows for sampling sequences; the final draw re-reads row n
    of both (one row for the bonus).  Invalid sequences are not counted.
    """
    s = w.elem_bytes
    V, K = w.V, w.K
    tot = 0
    for b, n in enumerate(np.asarray(accepted_len).tolist()):
        if n < 0:
            continue
        if w.greedy[b]:
            tot += (n + 1) * V * s
        else:
            tot += (n + 1) * V * s + min(n + 1, K) * V * s
            tot += (2 if n < K else 1) * V * s
    return tot



def reached_bytes(w: Workload, accepted_len: np.ndarray) -> int:
    """Bytes of logits the row statistics read when only reached positions are
    streamed: (n+1) target rows, plus min(n+1, K) draft rows for sampling
    sequences.  Invalid sequences (n = -1) count their first position only."""
    s = w.elem_bytes
    V, K = w.V, w.K
    tot = 0
    for b, n in enumerate(np.asarray(accepted_len).tolist()):
        m = max(n, 0)
        tot += (m + 1) * V * s
        if not w.greedy[b]:
            tot += min(m + 1, K) * V * s
    return tot


# ---------------------------------------------------------------------------
# Prompt-lookup workloads (no draft model).
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LookupWorkload:
    """Token histories for the proposer plus the target logits that verify
    its candidates (host side)."""
    name: str
    B: int
    K: int
    V: int
    dtype: int
    T: float
    history: np.ndarray      # [B, Lmax] int32 (row b valid up to hist_len[b])
    hist_len: np.ndarray     # [B] int32
    n_max: int
    n_min: int
    target: np.ndarray       # [B, K+1, V] stored logits
    uniforms: np.ndarray     # [B, K+1] fp32
    greedy: np.ndarray       # [B] uint8
    seed: int = 0


def synth_lookup(seed: int, B: int, K: int, V: int, Lmax: int, *, dtype: int, T: float = 1.0,
                 prompt_frac: float = 0.75, edit_rate: float = 0.02, agree: float = 0.8, bump: float = 12.0,
                 sigma: float = 3.0, n_max: int = 4, n_min: int = 1, greedy_mask: np.ndarray | None = None,
                 name: str = "lookup") -> LookupWorkload:
    """The code-editing pattern of a prompt-lookup workload: a prompt of
    Zipf(1.1)-distributed token ids, then an output that re-types a span of it,
    each copied token replaced by a random id with probability edit_rate.
    History lengths are drawn in [Lmax/2, Lmax].  Target logits follow the
    generic recipe (N(0, sigma) + the log-Zipf bias); at each of the first K
    positions, with probability `agree`, the token the copied span continues
    with gets `bump` added (a target that mostly agrees with the copy).  The
    generator knows that token from the span it copied, not from any proposer.
    """
    history = np.zeros((B, Lmax), np.int32)
    hist_len = np.zeros(B, np.int32)
    target = np.empty((B, K + 1, V), dtype={F32: np.float32, BF16: np.uint16}[dtype])
    uniforms = np.empty((B, K + 1), np.float32)
    greedy = np.zeros(B, np.uint8) if greedy_mask is None else greedy_mask.astype(np.uint8)
    bias = zipf_bias(V)
    pz = np.exp(bias.astype(np.float64))
    pz /= pz.sum()
    cz = np.cumsum(pz)
    seeds = _seq_seeds(seed, B, 4)

    def one(b):
        r_h, r_l, r_a, r_u = (np.random.Generator(np.random.PCG64(s)) for s in seeds[b])
        L = int(r_h.integers(max(2, Lmax // 2), Lmax + 1)) if Lmax >= 2 else Lmax
        P = max(1, int(L * prompt_frac))
        prompt = np.minimum(np.searchsorted(cz, r_h.random(P + K + 1)), V - 1).astype(np.int32)
        out_len = L - P
        start = int(r_h.integers(0, max(1, P - out_len)))
        src = prompt[start:start + out_len + K + 1]
        out = src[:out_len].copy()
        edits = r_h.random(out_len) < edit_rate
        out[edits] = r_h.integers(0, V, size=int(edits.sum()))
        h = np.concatenate([prompt[:P], out])[:L]
        history[b, :L] = h
        hist_len[b] = L
        l = r_l.standard_normal((K + 1, V), dtype=np.float32) * np.float32(sigma) + bias
        nxt = src[out_len:out_len + K]                  # what the copied span continues with
        for j in range(min(K, len(nxt))):
            if r_a.random() < agree:
                l[j, nxt[j]] += np.float32(bump)
        target[b] = _store(l, dtype)
        uniforms[b] = grid_uniforms(r_u, (K + 1,))

    with ThreadPoolExecutor(max_workers=min(_WORKERS, max(1, B))) as ex:
        list(ex.map(one, range(B)))
    return LookupWorkload(name=name, B=B, K=K, V=V, dtype=dtype, T=T, history=history, hist_len=hist_len,
                          n_max=n_max, n_min=n_min, target=target, uniforms=uniforms, greedy=greedy, seed=seed)


def lookup_152k(seed: int = 1005, B: int = 256) -> LookupWorkload:
    """B=256 histories of 2048-4096 tokens, K=8, V=152064 bf16, T=1, sampling."""
    return synth_lookup(seed, B, 8, 152064, 4096, dtype=BF16, name=f"lookup_B{B}_K8_V152064_L4096_bf16")
