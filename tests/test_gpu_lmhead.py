"""GPU parity of the fused LM head: repack, MFMA GEMM and the fused verify.

The GEMM is compared with the oracle's fp64 product of the same bf16 values.
Bound: bf16 x bf16 products are exact in fp32, and any order of d - 1 fp32
additions stays within d * 2^-24 * sum_k |h_k w_k| of the exact sum; the test
uses that worst-case bound (observed errors are far below it).
"""

import sys

import numpy as np
import pytest

import oracle
from oracle import parity
from speculative_sampling_verification_06_amd import binding
from speculative_sampling_verification_06_amd import inputs as I

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()
    oracle.build(force=False)
    return torch.device("cuda:0")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rand_bf16(rng, shape, scale):
    return I.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def _tiles(w):
    """W [d, V] as the header's packed layout, built by numpy indexing: tile
    (vt, kt) lane l element e = W[kt*16 + 8*(l//32) + e, vt*32 + l%32], the
    tiles ordered (vt // 8, kt, vt % 8).  Returns the layout and a mask of the
    elements the header defines (tiles past ceil(V/32) are not written)."""
    d, V = w.shape
    KT, G = -(-d // 16), -(-V // 256)
    pad = np.zeros((KT * 16, G * 256), dtype=w.dtype)
    pad[:d, :V] = w
    g, kt, j, l, e = np.meshgrid(np.arange(G), np.arange(KT), np.arange(8), np.arange(64), np.arange(8),
                                 indexing="ij")
    vt = g * 8 + j
    return pad[kt * 16 + 8 * (l // 32) + e, vt * 32 + l % 32].reshape(-1), (vt < -(-V // 32)).reshape(-1)


@pytest.mark.parametrize("d,V", [(1, 1), (70, 333), (4096, 130), (72, 64)])
def test_pack_layout(dev, d, V):
    import torch
    rng = np.random.default_rng(d + V)
    w = _rand_bf16(rng, (d, V), 1.0)
    pk = binding.lmhead_pack(binding.bf16_tensor(w, dev))
    torch.cuda.synchronize()
    got = pk.data.view(torch.int16).cpu().numpy().view(np.uint16)
    assert got.size * 2 == binding.packed_bytes(d, V)
    want, defined = _tiles(w)
    assert np.array_equal(got[defined], want[defined])


@pytest.mark.parametrize("M,d,V", [(1, 8, 1), (5, 24, 33), (192, 256, 1000), (200, 4096, 515),
                                   (37, 4104, 300), (192, 4096, 4100)])
def test_gemm_against_fp64_product(dev, M, d, V):
    import torch
    _log(f"[lmhead] gemm M={M} d={d} V={V}")
    rng = np.random.default_rng(M * 7 + d + V)
    h = _rand_bf16(rng, (M, d), 1.0)
    w = _rand_bf16(rng, (d, V), 0.02)
    wt = binding.lmhead_pack(binding.bf16_tensor(w, dev))
    got = binding.lmhead(binding.bf16_tensor(h, dev), wt)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    want = oracle.lmhead_logits(h.reshape(1, M, d), w)[0]
    habs = np.abs(I.bf16_bits_to_f32(h).astype(np.float64))
    wabs = np.abs(I.bf16_bits_to_f32(w).astype(np.float64))
    bound = d * U32 * (habs @ wabs)
    err = np.abs(got - want)
    _log(f"[lmhead] max err {err.max():.3g}, max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3g}")
    assert np.all(err <= bound)


def test_gemm_rejects_bad_shapes(dev):
    import torch
    h = torch.zeros(4, 12, dtype=torch.bfloat16, device=dev)
    pk = binding.PackedWeight(torch.zeros(binding.packed_bytes(12, 8) // 2, dtype=torch.bfloat16, device=dev),
                              12, 8)
    with pytest.raises(binding.SpecVerifyError):
        binding.lmhead(h, pk)          # d = 12 is not a multiple of 8


@pytest.mark.parametrize("mode,groups,la", [(binding.MODE_AUTO, 0, -1), (binding.MODE_EAGER, 0, -1),
                                             (binding.MODE_SEQ, 0, 0), (binding.MODE_SEQ, 0, 1),
                                             (binding.MODE_SEQ, 1, -1)],
                         ids=["auto", "eager", "seq", "seqla", "seq1"])
def test_fused_lmhead_verify_full_size(dev, mode, groups, la):
    binding.set_mode(mode)
    binding.set_seq_groups(groups)
    binding.set_seq_lookahead(la)
    try:
        _fused_case(dev)
    finally:
        binding.set_mode(binding.MODE_AUTO)
        binding.set_seq_groups(0)
        binding.set_seq_lookahead(-1)


@pytest.mark.parametrize("B,K,d,V", [(40, 4, 256, 1000), (7, 3, 72, 515), (3, 0, 64, 300)])
def test_lmhead_verify_greedy_ragged_invalid(dev, B, K, d, V):
    """Every other sequence greedy (its first proposals the target's argmax, so
    some are accepted), V not a multiple of 256 (a partial last column block),
    B*(K+1) above 192 (two row blocks) or not a multiple of 32, and two
    sequences with NaN hidden states at position 0 (invalid).  The oracle runs
    on the GPU's own fp32 logits, so greedy decisions must agree exactly."""
    import torch
    w = I.cfg_lmhead(seed=77 + B + V, B=B, K=K, d=d, V=V, draft_noise=0.3)
    w.greedy = (np.arange(B) % 2 == 0).astype(np.uint8)
    tgt64 = oracle.lmhead_logits(w.hidden, w.w_lm)
    tokens = w.tokens.copy()
    for b in range(0, B, 2):
        for j in range(min(K, b % (K + 2))):
            tokens[b, j] = int(np.argmax(tgt64[b, j]))
    w.tokens = tokens
    hidden = w.hidden.copy()
    if B >= 4:
        hidden[2, 0, d // 2] = 0x7FC0          # bf16 NaN: row 0 of a greedy sequence
        hidden[3, 0, 1] = 0x7FC0               # and of a sampling sequence
    w.hidden = hidden
    _log(f"[lmhead] greedy/ragged B={B} K={K} d={d} V={V}")
    d_h = binding.bf16_tensor(w.hidden, dev)
    wt = binding.lmhead_pack(binding.bf16_tensor(w.w_lm, dev))
    dd = binding.to_device(w, dev)
    out = binding.lmhead_verify(d_h, wt, dd["draft"], dd["tokens"], dd["uniforms"], w.T, dd["greedy"])
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    o = oracle.verify(w, target=g["target_logits"].astype(np.float64))
    rep = parity.compare(w, g, o)
    _log(f"[lmhead] parity {rep}; lengths {o.accepted_len.tolist()}")
    if B >= 4:
        assert g["accepted_len"][2] == -1 and g["accepted_len"][3] == -1
    assert (g["accepted_len"][0::2] > 0).any() or K == 0      # some greedy proposals accepted
    assert rep["flagged_mismatch"] == []


def _fused_case(dev):
    import torch
    w = I.cfg_lmhead()
    _log(f"[lmhead] {w.name}: generated")
    d_h = binding.bf16_tensor(w.hidden, dev)
    wt = binding.lmhead_pack(binding.bf16_tensor(w.w_lm, dev))
    dd = binding.to_device(w, dev)
    out = binding.lmhead_verify(d_h, wt, dd["draft"], dd["tokens"], dd["uniforms"], w.T, dd["greedy"])
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in out.items()}
    tgt64 = oracle.lmhead_logits(w.hidden, w.w_lm)
    err = np.abs(g["target_logits"].astype(np.float64) - tgt64)
    _log(f"[lmhead] logits max abs err {err.max():.3g}")
    o = oracle.verify(w, target=tgt64)
    rep = parity.compare(w, g, o)
    _log(f"[lmhead] verify parity {rep}")
    assert err.max() < 1e-3
    # near-uniform laws over 128k tokens (logits of std ~1.3 at T = 0.8): most
    # draws land on tokens narrower than 2e-5 and are flagged, so a differing
    # draw is allowed there (compare() already requires the flag); the other
    # named workloads assert none differ at all
    assert len(rep["flagged_mismatch"]) <= rep["flagged"], rep
