"""Thin Python binding of libspecverify.so (argument marshalling only).

Every step of the verify path runs in the HIP kernels behind the C ABI in
include/spec_verify.h.  torch supplies device memory and the stream; this
module only checks shapes and dtypes, passes data pointers and the current
stream, and keeps one zero-initialised workspace per device and stream.  There is no
CPU fallback: if the library is missing or no GPU is present, calls raise.
"""

from __future__ import annotations

import ctypes as C
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
SV_OK, SV_EINVAL, SV_EWORKSPACE, SV_ELAUNCH, SV_ESCRATCH = 0, -1, -2, -3, -4
SV_GAVE_UP = -2          # accepted_len of a sequence whose per-sequence wait gave up
SV_MAX_K = 63

# The exported names, as declared in include/spec_verify.h.
EXPORTS = ("sv_workspace_bytes", "spec_verify", "spec_verify_ex", "sv_stats", "sv_draw", "sv_lmhead_packed_bytes", "sv_lmhead_pack", "sv_lmhead",
           "sv_lmhead_verify_gemm", "sv_lmhead_verify_rest",
           "spec_lmhead_verify", "sv_sample_workspace_bytes", "sv_sample", "sv_kv_commit",
           "sv_set_mode", "sv_get_mode", "sv_schedule", "sv_set_seq_groups", "sv_seq_groups", "sv_set_wait_limit",
           "sv_set_seq_lookahead", "sv_seq_lookahead",
           "sv_lookup_propose", "spec_verify_lookup", "sv_last_hip_error",
           "spec_verify_noalloc", "sv_noalloc_scratch_bytes", "spec_verify_mode", "sv_strerror", "sv_version",
           "sv_hbm_probe", "sv_hbm_probe_words")
MODE_AUTO, MODE_EAGER, MODE_LAZY, MODE_SEQ = 0, 1, 2, 3


class SvDiag(C.Structure):
    _fields_ = [("p_tok", C.c_void_p), ("q_tok", C.c_void_p), ("lse_p", C.c_void_p),
                ("lse_q", C.c_void_p), ("res_mass", C.c_void_p)]


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        hip = None
        if code == SV_ELAUNCH and _lib is not None:
            hip = int(_lib.sv_last_hip_error())
        super().__init__(f"{msg} (code {code}" + (f", hipError_t {hip})" if hip is not None else ")"))
        self.code = code
        self.hip_error = hip


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load the HIP library (no GPU needed to load it).

    PyTorch-ROCm brings its own HIP runtime under the same soname; loaded
    first, ours would pull a second runtime into the process, which then sees
    no device.  So torch, when installed, is imported before the library, and
    the library binds to the runtime torch already loaded."""
    global _lib
    with _lock:
        if _lib is None:
            try:
                import torch  # noqa: F401  (one HIP runtime per process)
            except ImportError:
                pass
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with "
                    "`python -m speculative_sampling_verification_06_amd.build`")
            lib = C.CDLL(path)
            verify_args = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_float, C.c_void_p,
                           C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                           C.POINTER(SvDiag), C.c_void_p, C.c_size_t, C.c_void_p]
            for name in ("spec_verify", "sv_stats", "sv_draw"):
                fn = getattr(lib, name)
                fn.restype = C.c_int
                fn.argtypes = verify_args
            lib.spec_verify_mode.restype = C.c_int
            lib.spec_verify_mode.argtypes = [C.c_int] + verify_args
            lib.spec_verify_noalloc.restype = C.c_int
            lib.spec_verify_noalloc.argtypes = verify_args[:13] + [C.c_void_p]
            lib.sv_noalloc_scratch_bytes.restype = C.c_size_t
            lib.sv_noalloc_scratch_bytes.argtypes = []
            lib.spec_verify_ex.restype = C.c_int
            lib.spec_verify_ex.argtypes = verify_args[:10] + [C.c_int32] + verify_args[10:]
            lib.sv_workspace_bytes.restype = C.c_size_t
            lib.sv_workspace_bytes.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32]
            lib.sv_strerror.restype = C.c_char_p
            lib.sv_strerror.argtypes = [C.c_int]
            lib.sv_version.restype = C.c_int
            lib.sv_version.argtypes = []
            lib.sv_sample_workspace_bytes.restype = C.c_size_t
            lib.sv_sample_workspace_bytes.argtypes = [C.c_int32, C.c_int32, C.c_int32]
            lib.sv_sample.restype = C.c_int
            lib.sv_sample.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_float, C.c_void_p, C.c_int32,
                                      C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
            lib.sv_kv_commit.restype = C.c_int
            lib.sv_kv_commit.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_int32, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]
            lib.sv_last_hip_error.restype = C.c_int
            lib.sv_last_hip_error.argtypes = []
            lib.sv_hbm_probe.restype = C.c_int
            lib.sv_hbm_probe.argtypes = [C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
            lib.sv_hbm_probe_words.restype = C.c_int32
            lib.sv_hbm_probe_words.argtypes = []
            lib.sv_lookup_propose.restype = C.c_int
            lib.sv_lookup_propose.argtypes = [C.c_void_p, C.c_void_p] + [C.c_int32] * 5 + [C.c_void_p] * 3
            lib.spec_verify_lookup.restype = C.c_int
            lib.spec_verify_lookup.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                               C.c_float, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                               C.c_void_p, C.c_void_p, C.POINTER(SvDiag), C.c_void_p,
                                               C.c_size_t, C.c_void_p]
            lib.sv_set_mode.restype = C.c_int
            lib.sv_set_mode.argtypes = [C.c_int]
            lib.sv_get_mode.restype = C.c_int
            lib.sv_get_mode.argtypes = []
            lib.sv_schedule.restype = C.c_int
            lib.sv_schedule.argtypes = [C.c_int32] * 5
            lib.sv_set_seq_groups.restype = C.c_int
            lib.sv_set_seq_groups.argtypes = [C.c_int]
            lib.sv_seq_groups.restype = C.c_int
            lib.sv_seq_groups.argtypes = [C.c_int32] * 5
            lib.sv_set_seq_lookahead.restype = C.c_int
            lib.sv_set_seq_lookahead.argtypes = [C.c_int]
            lib.sv_seq_lookahead.restype = C.c_int
            lib.sv_seq_lookahead.argtypes = [C.c_int32] * 5
            lib.sv_set_wait_limit.restype = C.c_int
            lib.sv_set_wait_limit.argtypes = [C.c_int32]
            lib.sv_lmhead_packed_bytes.restype = C.c_size_t
            lib.sv_lmhead_packed_bytes.argtypes = [C.c_int32, C.c_int32]
            lib.sv_lmhead_pack.restype = C.c_int
            lib.sv_lmhead_pack.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]
            lib.sv_lmhead.restype = C.c_int
            lib.sv_lmhead.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                      C.c_void_p]
            lmv_args = [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                        C.c_void_p, C.c_float, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                        C.c_void_p, C.POINTER(SvDiag), C.c_void_p, C.c_size_t, C.c_void_p]
            for name in ("spec_lmhead_verify", "sv_lmhead_verify_gemm", "sv_lmhead_verify_rest"):
                getattr(lib, name).restype = C.c_int
                getattr(lib, name).argtypes = lmv_args
            _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load_library().sv_strerror(int(code)).decode()


def workspace_bytes(B: int, K: int, V: int, dtype: int) -> int:
    return int(load_library().sv_workspace_bytes(B, K, V, dtype))


def set_mode(mode: int) -> None:
    """Row-statistics schedule for later calls: MODE_AUTO, MODE_EAGER, MODE_LAZY or MODE_SEQ."""
    rc = load_library().sv_set_mode(int(mode))
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))


def get_mode() -> int:
    return int(load_library().sv_get_mode())


def set_seq_groups(groups: int) -> None:
    """Cap on workgroups per sequence under MODE_SEQ (0 = as many as the device holds)."""
    rc = load_library().sv_set_seq_groups(int(groups))
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))


def set_seq_lookahead(lookahead: int) -> None:
    """Lookahead of MODE_SEQ: -1 = by shape (default), 0 or 1 to force it."""
    rc = load_library().sv_set_seq_lookahead(int(lookahead))
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))


def seq_lookahead(B: int, K: int, V: int, target_dtype: int, draft_dtype=None) -> int:
    """Lookahead a MODE_SEQ call of this shape would use (0: none, or not MODE_SEQ)."""
    rc = int(load_library().sv_seq_lookahead(B, K, V, target_dtype,
                                             target_dtype if draft_dtype is None else draft_dtype))
    if rc < 0:
        raise SpecVerifyError(rc, strerror(rc))
    return rc


def set_wait_limit(polls: int) -> None:
    """Polls before a wait of the MODE_SEQ exchange gives up (0 = the default, 2**20)."""
    rc = load_library().sv_set_wait_limit(int(polls))
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))


def seq_groups(B: int, K: int, V: int, target_dtype: int, draft_dtype=None) -> int:
    """Workgroups per sequence a MODE_SEQ call of this shape would use (0: not MODE_SEQ)."""
    rc = int(load_library().sv_seq_groups(B, K, V, target_dtype,
                                          target_dtype if draft_dtype is None else draft_dtype))
    if rc < 0:
        raise SpecVerifyError(rc, strerror(rc))
    return rc


def schedule(B: int, K: int, V: int, target_dtype: int, draft_dtype=None) -> int:
    """MODE_EAGER, MODE_LAZY or MODE_SEQ: what a verify call of this shape would run."""
    rc = int(load_library().sv_schedule(B, K, V, target_dtype, target_dtype if draft_dtype is None else draft_dtype))
    if rc < 0:
        raise SpecVerifyError(rc, strerror(rc))
    return rc


# ------------------------------------------------------------------ torch --

def _torch():
    import torch
    return torch


_ws_cache: dict = {}


def get_workspace(nbytes: int, device, stream=None):
    """A zero-initialised workspace of at least nbytes on `device`, reused by
    the calls on one stream (raw HIP stream handle; None = the current one):
    calls sharing a workspace must be ordered, and calls on different streams
    may overlap, so each stream gets its own."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    key = (str(device), int(stream or 0))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        # allocated on the stream that uses it, so the caching allocator hands a
        # replaced workspace's memory out again only in that stream's order
        # (the kernels of earlier calls on it may still be reading the old one)
        with torch.cuda.stream(torch.cuda.ExternalStream(int(stream or 0), device=device)):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _dev_ptr(t, name, dtype=None, shape=None):
    if t is None:
        return None
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr() if t.numel() else None


class Outputs(dict):
    __getattr__ = dict.__getitem__


def _call(fn_name, target, draft, tokens, uniforms, temperature, greedy=None, *,
          outputs=None, diag=True, workspace=None, stream=None, mode=None):
    torch = _torch()
    lib = load_library()
    if target.dim() != 3:
        raise ValueError("target logits must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dt = _dtype_code(target)
    dev = target.device
    _dev_ptr(target, "target_logits", shape=(B, K + 1, V))
    ddt = dt
    if draft is not None:
        ddt = _dtype_code(draft)
        if ddt != dt and fn_name != "spec_verify":
            raise TypeError("sv_stats / sv_draw need one storage type for target and draft logits")
        _dev_ptr(draft, "draft_logits", shape=(B, K, V))
    if tokens is not None:
        _dev_ptr(tokens, "draft_tokens", torch.int32, (B, K))
    _dev_ptr(uniforms, "uniforms", torch.float32, (B, K + 1))
    if greedy is not None:
        _dev_ptr(greedy, "greedy_flag", torch.uint8, (B,))
    if outputs is None:
        outputs = Outputs(
            accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
            out_tokens=torch.empty(B, K + 1, dtype=torch.int32, device=dev))
        if diag:
            outputs.update(
                p_tok=torch.empty(B, K, dtype=torch.float32, device=dev),
                q_tok=torch.empty(B, K, dtype=torch.float32, device=dev),
                lse_p=torch.empty(B, K + 1, dtype=torch.float32, device=dev),
                lse_q=torch.empty(B, K, dtype=torch.float32, device=dev),
                res_mass=torch.empty(B, dtype=torch.float32, device=dev))
    dg = None
    if "p_tok" in outputs:
        dg = SvDiag(*[_dev_ptr(outputs[k], k) for k in ("p_tok", "q_tok", "lse_p", "lse_q", "res_mass")])
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    noalloc = fn_name == "spec_verify_noalloc"
    if noalloc:
        if ddt != dt:
            raise TypeError("spec_verify_noalloc needs one storage type for target and draft logits")
        ws_args = ()
    else:
        need = lib.sv_workspace_bytes(B, K, V, dt)
        ws = workspace if workspace is not None else get_workspace(need, dev, stream)
        ws_args = (ws.data_ptr(), ws.numel())
    dts = (dt,) if ddt == dt else (dt, ddt)
    if ddt != dt:
        if mode is not None:
            raise TypeError("a per-call schedule needs one storage type for target and draft logits")
        fn_name = "spec_verify_ex"
    lead = ()
    if mode is not None:
        if fn_name != "spec_verify":
            raise TypeError("a per-call schedule applies to the whole verify step only")
        fn_name, lead = "spec_verify_mode", (int(mode),)
    rc = getattr(lib, fn_name)(*lead,
        target.data_ptr(), None if draft is None else draft.data_ptr(),
        None if tokens is None or tokens.numel() == 0 else tokens.data_ptr(),
        uniforms.data_ptr(), C.c_float(float(temperature)),
        None if greedy is None else greedy.data_ptr(), B, K, V, *dts,
        _dev_ptr(outputs["accepted_len"], "accepted_len", torch.int32, (B,)),
        _dev_ptr(outputs["out_tokens"], "out_tokens", torch.int32, (B, K + 1)),
        None if dg is None else C.byref(dg), *ws_args, stream)
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))
    return outputs


def verify(target, draft, tokens, uniforms, temperature, greedy=None, **kw):
    """spec_verify on torch device tensors -> Outputs(accepted_len, out_tokens[, diagnostics]).
    mode=MODE_* (keyword) picks the schedule for this call only (spec_verify_mode)."""
    return _call("spec_verify", target, draft, tokens, uniforms, temperature, greedy, **kw)


def verify_noalloc(target, draft, tokens, uniforms, temperature, greedy=None, **kw):
    """spec_verify_noalloc: spec_verify with the library's static scratch as its
    workspace (the library allocates nothing; outputs are allocated here
    unless passed in `outputs`)."""
    if "workspace" in kw:
        raise TypeError("spec_verify_noalloc takes no workspace")
    return _call("spec_verify_noalloc", target, draft, tokens, uniforms, temperature, greedy, **kw)


def noalloc_scratch_bytes() -> int:
    return int(load_library().sv_noalloc_scratch_bytes())


def stats(target, draft, tokens, uniforms, temperature, greedy=None, **kw):
    """First launch only (row statistics, tests, first rejection, greedy results)."""
    return _call("sv_stats", target, draft, tokens, uniforms, temperature, greedy, **kw)


def draw(target, draft, tokens, uniforms, temperature, greedy=None, **kw):
    """Second launch only (final draw of sampling sequences); pass stats()'s outputs."""
    return _call("sv_draw", target, draft, tokens, uniforms, temperature, greedy, **kw)


def to_device(w, device="cuda:0"):
    """Copy a host Workload's arrays to device tensors (bf16 bits become torch.bfloat16)."""
    torch = _torch()
    import numpy as np

    def logits(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        if a.dtype == np.float32:
            return torch.from_numpy(a).to(device)
        raise TypeError(f"unsupported logit storage {a.dtype} for the device path")

    return dict(
        target=logits(w.target) if w.target.size else None,
        draft=logits(w.draft) if w.K > 0 else None,
        tokens=torch.from_numpy(np.ascontiguousarray(w.tokens, np.int32)).to(device),
        uniforms=torch.from_numpy(np.ascontiguousarray(w.uniforms, np.float32)).to(device),
        greedy=torch.from_numpy(np.ascontiguousarray(w.greedy, np.uint8)).to(device),
        temperature=float(w.T))


class Bound:
    """One verify problem bound to fixed device tensors: the C arguments are
    marshalled once, so each call is a single ctypes call (a few microseconds
    of host time) and back-to-back launches keep the GPU busy.

    Checks happen in the constructor (the same checks as verify()); the
    tensors must stay alive and keep their shapes while the object is used.
    """

    def __init__(self, target, draft, tokens, uniforms, temperature, greedy=None, *,
                 outputs=None, diag=True, stream=None):
        torch = _torch()
        mixed = draft is not None and draft.dtype != target.dtype
        # one checked call builds the outputs and the workspace
        self.outputs = _call("spec_verify" if mixed else "sv_stats", target, draft, tokens, uniforms,
                             temperature, greedy, outputs=outputs, diag=diag, stream=stream)
        torch.cuda.synchronize(target.device)
        lib = load_library()
        B, K1, V = target.shape
        K = K1 - 1
        dt = _dtype_code(target)
        dts = (C.c_int32(dt),) if not mixed else (C.c_int32(dt), C.c_int32(_dtype_code(draft)))
        o = self.outputs
        self._dg = None
        if "p_tok" in o:
            self._dg = SvDiag(*[_dev_ptr(o[k], k) for k in ("p_tok", "q_tok", "lse_p", "lse_q", "res_mass")])
        if stream is None:
            stream = torch.cuda.current_stream(target.device).cuda_stream
        ws = get_workspace(lib.sv_workspace_bytes(B, K, V, dt), target.device, stream)
        self._keep = (target, draft, tokens, uniforms, greedy, ws)
        self._args = (
            C.c_void_p(target.data_ptr()), C.c_void_p(None if draft is None else draft.data_ptr()),
            C.c_void_p(None if tokens is None or tokens.numel() == 0 else tokens.data_ptr()),
            C.c_void_p(uniforms.data_ptr()), C.c_float(float(temperature)),
            C.c_void_p(None if greedy is None else greedy.data_ptr()),
            C.c_int32(B), C.c_int32(K), C.c_int32(V), *dts,
            C.c_void_p(o["accepted_len"].data_ptr()), C.c_void_p(o["out_tokens"].data_ptr()),
            None if self._dg is None else C.byref(self._dg),
            C.c_void_p(ws.data_ptr()), C.c_size_t(ws.numel()), C.c_void_p(stream))
        self.mixed = mixed
        if mixed:
            self._verify, self._stats, self._draw = lib.spec_verify_ex, None, None
        else:
            self._verify, self._stats, self._draw = lib.spec_verify, lib.sv_stats, lib.sv_draw

    def _check(self, rc):
        if rc != SV_OK:
            raise SpecVerifyError(rc, strerror(rc))

    def verify(self):
        self._check(self._verify(*self._args))
        return self.outputs

    def stats(self):
        if self._stats is None:
            raise TypeError("the split launches need one storage type for target and draft logits")
        self._check(self._stats(*self._args))
        return self.outputs

    def draw(self):
        if self._draw is None:
            raise TypeError("the split launches need one storage type for target and draft logits")
        self._check(self._draw(*self._args))
        return self.outputs


class BoundLMHead:
    """The LM-head GEMM of one problem with pre-marshalled arguments."""

    def __init__(self, hidden2d, packed, logits2d, stream=None):
        torch = _torch()
        M, d = hidden2d.shape
        V = packed.V
        _dev_ptr(hidden2d, "hidden", torch.bfloat16, (M, d))
        _check_packed(packed, d)
        _dev_ptr(logits2d, "logits", torch.float32, (M, V))
        if stream is None:
            stream = torch.cuda.current_stream(hidden2d.device).cuda_stream
        self._keep = (hidden2d, packed, logits2d)
        self._fn = load_library().sv_lmhead
        self._args = (C.c_void_p(hidden2d.data_ptr()), C.c_void_p(packed.data.data_ptr()), C.c_int32(M), C.c_int32(d),
                      C.c_int32(V), C.c_void_p(logits2d.data_ptr()), C.c_void_p(stream))

    def __call__(self):
        _check_rc(self._fn(*self._args))


# ---------------------------------------------------------------- LM head --

def _check_rc(rc):
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))


class PackedWeight:
    """The LM-head weight W [d, V] in the GEMM's tiled layout (sv_lmhead_pack):
    `data` is a 1-D bf16 device tensor of sv_lmhead_packed_bytes(d, V) bytes."""

    def __init__(self, data, d, V):
        self.data, self.d, self.V = data, int(d), int(V)


def packed_bytes(d, V):
    """sv_lmhead_packed_bytes: size of the tiled weight for W [d, V] (0 if d or V < 1)."""
    return int(load_library().sv_lmhead_packed_bytes(d, V))


def _check_packed(packed, d):
    torch = _torch()
    if not isinstance(packed, PackedWeight):
        raise TypeError("the LM-head weight must be the PackedWeight that lmhead_pack returns")
    if packed.d != d:
        raise ValueError(f"hidden size {d} does not match the packed weight's {packed.d}")
    _dev_ptr(packed.data, "packed weight", torch.bfloat16, (packed_bytes(packed.d, packed.V) // 2,))


def lmhead_pack(w_dv, out=None):
    """One-time repack of the static LM-head weight W [d, V] bf16 into the
    GEMM's tiled layout; returns a PackedWeight (its data in `out` if given)."""
    torch = _torch()
    d, V = w_dv.shape
    _dev_ptr(w_dv, "w_dv", torch.bfloat16, (d, V))
    n = packed_bytes(d, V) // 2
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=w_dv.device)
    _dev_ptr(out, "packed weight", torch.bfloat16, (n,))
    _check_rc(load_library().sv_lmhead_pack(w_dv.data_ptr(), out.data_ptr(), d, V,
                                            torch.cuda.current_stream(w_dv.device).cuda_stream))
    return PackedWeight(out, d, V)


def lmhead(hidden, packed, out=None):
    """logits [M, V] fp32 = hidden [M, d] bf16 x W, W given packed (lmhead_pack)."""
    torch = _torch()
    M, d = hidden.shape
    V = packed.V
    _dev_ptr(hidden, "hidden", torch.bfloat16, (M, d))
    _check_packed(packed, d)
    if out is None:
        out = torch.empty(M, V, dtype=torch.float32, device=hidden.device)
    _dev_ptr(out, "logits", torch.float32, (M, V))
    _check_rc(load_library().sv_lmhead(hidden.data_ptr(), packed.data.data_ptr(), M, d, V, out.data_ptr(),
                                       torch.cuda.current_stream(hidden.device).cuda_stream))
    return out


class BoundLMHeadVerify:
    """spec_lmhead_verify of one problem with pre-marshalled arguments; also
    its two parts (sv_lmhead_verify_gemm, sv_lmhead_verify_rest) for timing."""

    def __init__(self, hidden, packed, draft, tokens, uniforms, temperature, greedy=None, *, diag=True,
                 stream=None):
        torch = _torch()
        self.outputs, self._args, self._keep = _lmhead_verify_call(hidden, packed, draft, tokens, uniforms,
                                                                   temperature, greedy, diag=diag, stream=stream)
        torch.cuda.synchronize(hidden.device)
        lib = load_library()
        self._all, self._gemm, self._rest = lib.spec_lmhead_verify, lib.sv_lmhead_verify_gemm, lib.sv_lmhead_verify_rest

    def __call__(self):
        _check_rc(self._all(*self._args))
        return self.outputs

    def gemm(self):
        _check_rc(self._gemm(*self._args))

    def rest(self):
        _check_rc(self._rest(*self._args))
        return self.outputs


def lmhead_verify(hidden, packed, draft, tokens, uniforms, temperature, greedy=None, *,
                  target_logits=None, diag=True, stream=None):
    """spec_lmhead_verify: the LM-head GEMM into target_logits [B, K+1, V] fp32,
    then the verify step.  Returns Outputs (+ target_logits)."""
    return _lmhead_verify_call(hidden, packed, draft, tokens, uniforms, temperature, greedy,
                               target_logits=target_logits, diag=diag, stream=stream)[0]


def _lmhead_verify_call(hidden, packed, draft, tokens, uniforms, temperature, greedy=None, *,
                        target_logits=None, diag=True, stream=None):
    torch = _torch()
    lib = load_library()
    B, K1, d = hidden.shape
    K = K1 - 1
    V = packed.V
    dev = hidden.device
    _dev_ptr(hidden, "hidden", torch.bfloat16, (B, K + 1, d))
    _check_packed(packed, d)
    if draft is not None:
        _dev_ptr(draft, "draft_logits", shape=(B, K, V))
    if target_logits is None:
        target_logits = torch.empty(B, K + 1, V, dtype=torch.float32, device=dev)
    _dev_ptr(target_logits, "target_logits", torch.float32, (B, K + 1, V))
    if tokens is not None:
        _dev_ptr(tokens, "draft_tokens", torch.int32, (B, K))
    _dev_ptr(uniforms, "uniforms", torch.float32, (B, K + 1))
    o = Outputs(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                out_tokens=torch.empty(B, K + 1, dtype=torch.int32, device=dev))
    dg = None
    if diag:
        o.update(p_tok=torch.empty(B, K, device=dev), q_tok=torch.empty(B, K, device=dev),
                 lse_p=torch.empty(B, K + 1, device=dev), lse_q=torch.empty(B, K, device=dev),
                 res_mass=torch.empty(B, device=dev))
        dg = SvDiag(*[o[k].data_ptr() for k in ("p_tok", "q_tok", "lse_p", "lse_q", "res_mass")])
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ws = get_workspace(lib.sv_workspace_bytes(B, K, V, SV_F32), dev, stream)
    ddt = SV_F32 if draft is None else _dtype_code(draft)
    args = (C.c_void_p(hidden.data_ptr()), C.c_void_p(packed.data.data_ptr()), C.c_int32(d),
            C.c_void_p(target_logits.data_ptr()), C.c_void_p(None if draft is None else draft.data_ptr()),
            C.c_int32(ddt), C.c_void_p(None if tokens is None or tokens.numel() == 0 else tokens.data_ptr()),
            C.c_void_p(uniforms.data_ptr()), C.c_float(float(temperature)),
            C.c_void_p(None if greedy is None else greedy.data_ptr()), C.c_int32(B), C.c_int32(K), C.c_int32(V),
            C.c_void_p(o["accepted_len"].data_ptr()), C.c_void_p(o["out_tokens"].data_ptr()),
            None if dg is None else C.byref(dg), C.c_void_p(ws.data_ptr()), C.c_size_t(ws.numel()),
            C.c_void_p(stream))
    _check_rc(lib.spec_lmhead_verify(*args))
    o["target_logits"] = target_logits
    return o, args, (hidden, packed, draft, tokens, uniforms, greedy, ws, target_logits, dg)


def bf16_tensor(bits, device):
    """A torch bfloat16 device tensor from uint16 bf16 bits (numpy)."""
    torch = _torch()
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


# ------------------------------------------------------- draft-side sampling --

def sample(logits, uniforms, temperature, greedy=None, *, lse=False, stream=None):
    """x ~ softmax(logits / T) per row of logits [B, V] (argmax for greedy rows).

    Returns tokens [B] int32 (-1 for an invalid row), and lse [B] if asked."""
    torch = _torch()
    lib = load_library()
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    B, V = logits.shape
    dt = _dtype_code(logits)
    dev = logits.device
    _dev_ptr(logits, "logits", shape=(B, V))
    _dev_ptr(uniforms, "uniforms", torch.float32, (B,))
    if greedy is not None:
        _dev_ptr(greedy, "greedy_flag", torch.uint8, (B,))
    tokens = torch.empty(B, dtype=torch.int32, device=dev)
    out_lse = torch.empty(B, dtype=torch.float32, device=dev) if lse else None
    need = lib.sv_sample_workspace_bytes(B, V, dt)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ws = get_workspace(need, dev, stream)
    _check_rc(lib.sv_sample(logits.data_ptr() if B else None, dt, uniforms.data_ptr() if B else None,
                            C.c_float(float(temperature)), None if greedy is None else greedy.data_ptr(), B, V,
                            tokens.data_ptr() if B else None, None if out_lse is None else out_lse.data_ptr(),
                            ws.data_ptr(), ws.numel(), stream))
    return (tokens, out_lse) if lse else tokens


# ------------------------------------------------------------ prompt lookup --

def lookup_propose(history, hist_len, n_max, n_min, K, *, cand=None, klen=None, stream=None):
    """Candidates from the history [B, Lmax] int32 (hist_len [B] int32 tokens per row):
    returns (cand [B, K] int32 padded with -1, klen [B] int32)."""
    torch = _torch()
    B, Lmax = history.shape
    dev = history.device
    _dev_ptr(history, "history", torch.int32, (B, Lmax))
    _dev_ptr(hist_len, "hist_len", torch.int32, (B,))
    if cand is None:
        cand = torch.empty(B, K, dtype=torch.int32, device=dev)
    if klen is None:
        klen = torch.empty(B, dtype=torch.int32, device=dev)
    _dev_ptr(cand, "cand", torch.int32, (B, K))
    _dev_ptr(klen, "klen", torch.int32, (B,))
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _check_rc(load_library().sv_lookup_propose(
        history.data_ptr() if history.numel() else None, hist_len.data_ptr() if B else None, B, Lmax,
        int(n_max), int(n_min), int(K), cand.data_ptr() if cand.numel() else None,
        klen.data_ptr() if B else None, stream))
    return cand, klen


def verify_lookup(target, cand, klen, uniforms, temperature, greedy=None, *, diag=True, workspace=None,
                  stream=None):
    """spec_verify_lookup: the verify step on prompt-lookup candidates (one-hot proposals)."""
    torch = _torch()
    lib = load_library()
    if target.dim() != 3:
        raise ValueError("target logits must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dt = _dtype_code(target)
    dev = target.device
    _dev_ptr(target, "target_logits", shape=(B, K + 1, V))
    _dev_ptr(cand, "cand", torch.int32, (B, K))
    _dev_ptr(klen, "klen", torch.int32, (B,))
    _dev_ptr(uniforms, "uniforms", torch.float32, (B, K + 1))
    if greedy is not None:
        _dev_ptr(greedy, "greedy_flag", torch.uint8, (B,))
    outputs = Outputs(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
                      out_tokens=torch.empty(B, K + 1, dtype=torch.int32, device=dev))
    dg = None
    if diag:
        outputs.update(p_tok=torch.empty(B, K, dtype=torch.float32, device=dev),
                       q_tok=torch.empty(B, K, dtype=torch.float32, device=dev),
                       lse_p=torch.empty(B, K + 1, dtype=torch.float32, device=dev),
                       lse_q=torch.empty(B, K, dtype=torch.float32, device=dev),
                       res_mass=torch.empty(B, dtype=torch.float32, device=dev))
        dg = SvDiag(*[_dev_ptr(outputs[k], k) for k in ("p_tok", "q_tok", "lse_p", "lse_q", "res_mass")])
    need = lib.sv_workspace_bytes(B, K, V, dt)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ws = workspace if workspace is not None else get_workspace(need, dev, stream)
    _check_rc(lib.spec_verify_lookup(
        target.data_ptr() if B else None, dt, _dev_ptr(cand, "cand"), _dev_ptr(klen, "klen"),
        _dev_ptr(uniforms, "uniforms"), C.c_float(float(temperature)), _dev_ptr(greedy, "greedy_flag"), B, K, V,
        _dev_ptr(outputs["accepted_len"], "accepted_len"), _dev_ptr(outputs["out_tokens"], "out_tokens"),
        None if dg is None else C.byref(dg), ws.data_ptr(), ws.numel(), stream))
    return outputs


class BoundLookup:
    """Prompt lookup bound to fixed device tensors: propose() fills cand/klen
    from the history, verify() runs spec_verify_lookup on them; each is one
    pre-marshalled ctypes call."""

    def __init__(self, history, hist_len, n_max, n_min, target, uniforms, temperature, greedy=None, *,
                 diag=True, stream=None):
        torch = _torch()
        lib = load_library()
        B, K1, V = target.shape
        K = K1 - 1
        self.cand, self.klen = lookup_propose(history, hist_len, n_max, n_min, K, stream=stream)
        self.outputs = verify_lookup(target, self.cand, self.klen, uniforms, temperature, greedy, diag=diag,
                                     stream=stream)
        torch.cuda.synchronize(target.device)
        dt = _dtype_code(target)
        o = self.outputs
        self._dg = None
        if "p_tok" in o:
            self._dg = SvDiag(*[_dev_ptr(o[k], k) for k in ("p_tok", "q_tok", "lse_p", "lse_q", "res_mass")])
        if stream is None:
            stream = torch.cuda.current_stream(target.device).cuda_stream
        ws = get_workspace(lib.sv_workspace_bytes(B, K, V, dt), target.device, stream)
        self._keep = (history, hist_len, target, uniforms, greedy, ws)
        Lmax = history.shape[1]
        self._pargs = (C.c_void_p(_dev_ptr(history, "history")), C.c_void_p(_dev_ptr(hist_len, "hist_len")),
                       C.c_int32(B), C.c_int32(Lmax), C.c_int32(n_max), C.c_int32(n_min), C.c_int32(K),
                       C.c_void_p(_dev_ptr(self.cand, "cand")), C.c_void_p(_dev_ptr(self.klen, "klen")),
                       C.c_void_p(stream))
        self._vargs = (C.c_void_p(target.data_ptr()), C.c_int32(dt), C.c_void_p(_dev_ptr(self.cand, "cand")),
                       C.c_void_p(_dev_ptr(self.klen, "klen")), C.c_void_p(uniforms.data_ptr()),
                       C.c_float(float(temperature)), C.c_void_p(_dev_ptr(greedy, "greedy_flag")),
                       C.c_int32(B), C.c_int32(K), C.c_int32(V),
                       C.c_void_p(o["accepted_len"].data_ptr()), C.c_void_p(o["out_tokens"].data_ptr()),
                       None if self._dg is None else C.byref(self._dg),
                       C.c_void_p(ws.data_ptr()), C.c_size_t(ws.numel()), C.c_void_p(stream))
        self._propose, self._verify = lib.sv_lookup_propose, lib.spec_verify_lookup

    def propose(self):
        _check_rc(self._propose(*self._pargs))
        return self.cand, self.klen

    def verify(self):
        _check_rc(self._verify(*self._vargs))
        return self.outputs


# --------------------------------------------------------------- KV commit --

def kv_commit(cache, cache_len, staged, accepted_len, offset=1, status=None, stream=None):
    """Commit the accepted prefix: cache [P, B, L, ...], cache_len [B] int32 (updated in place),
    staged [P, B, K + offset, ...] (or None: entries already written in place),
    accepted_len [B] int32.  The trailing dims of cache and staged are one row (any dtype).
    Returns status [B] int32 (0 committed, 1 invalid, 2 would overflow)."""
    torch = _torch()
    P, B, L = cache.shape[:3]
    row_bytes = cache[0, 0, 0].numel() * cache.element_size() if L else 0
    _dev_ptr(cache, "cache")
    _dev_ptr(cache_len, "cache_len", torch.int32, (B,))
    _dev_ptr(accepted_len, "accepted_len", torch.int32, (B,))
    if staged is not None:
        _dev_ptr(staged, "staged")
        srow = 1
        for n in staged.shape[3:]:
            srow *= n
        if staged.dim() != cache.dim() or staged.shape[0] != P or staged.shape[1] != B or \
                staged.dtype != cache.dtype or srow * staged.element_size() != row_bytes:
            raise ValueError("staged must be [P, B, K + offset, row] like the cache")
        K = staged.shape[2] - offset
    else:
        raise ValueError("give K through staged, or use kv_commit_in_place")
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=cache.device)
    if stream is None:
        stream = torch.cuda.current_stream(cache.device).cuda_stream
    _check_rc(load_library().sv_kv_commit(cache.data_ptr(), cache_len.data_ptr(), staged.data_ptr(),
                                          accepted_len.data_ptr(), P, B, K, offset, L, row_bytes,
                                          status.data_ptr(), stream))
    return status


def kv_commit_in_place(cache_len, accepted_len, K, offset=1, l_max=None, status=None, stream=None):
    """The in-place variant: entries already sit at [len, len + K + offset); only lengths change."""
    torch = _torch()
    B = cache_len.shape[0]
    _dev_ptr(cache_len, "cache_len", torch.int32, (B,))
    _dev_ptr(accepted_len, "accepted_len", torch.int32, (B,))
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=cache_len.device)
    if stream is None:
        stream = torch.cuda.current_stream(cache_len.device).cuda_stream
    _check_rc(load_library().sv_kv_commit(None, cache_len.data_ptr(), None, accepted_len.data_ptr(), 1, B, K,
                                          offset, int(l_max if l_max is not None else 2 ** 62), 1,
                                          status.data_ptr(), stream))
    return status



PROBE_READ, PROBE_COPY = 0, 1


def hbm_probe(kind, src, dst=None, stream=None):
    """sv_hbm_probe: a plain streaming read (kind PROBE_READ; dst, if given,
    holds sv_hbm_probe_words() int32 words) or copy (PROBE_COPY; dst like src)
    over the whole of src, a contiguous device tensor.  Returns dst."""
    torch = _torch()
    _dev_ptr(src, "src")
    nbytes = src.numel() * src.element_size()
    lib = load_library()
    if dst is None:
        if kind == PROBE_READ:
            words = int(lib.sv_hbm_probe_words())
            if words < 1:
                raise RuntimeError("sv_hbm_probe_words: device not queryable")
            dst = torch.empty(words, dtype=torch.int32, device=src.device)
        else:
            dst = torch.empty_like(src)
    _dev_ptr(dst, "dst")
    need = 4 * int(lib.sv_hbm_probe_words()) if kind == PROBE_READ else nbytes
    if dst.numel() * dst.element_size() < need:
        raise ValueError(f"dst holds {dst.numel() * dst.element_size()} bytes, needs {need}")
    if stream is None:
        stream = torch.cuda.current_stream(src.device).cuda_stream
    _check_rc(lib.sv_hbm_probe(kind, src.data_ptr(), dst.data_ptr(), nbytes, stream))
    return dst


class BoundSample:
    """sv_sample on fixed tensors with pre-marshalled arguments."""

    def __init__(self, logits, uniforms, temperature, greedy=None, stream=None):
        torch = _torch()
        self.tokens = sample(logits, uniforms, temperature, greedy)       # checked once
        B, V = logits.shape
        dt = _dtype_code(logits)
        lib = load_library()
        if stream is None:
            stream = torch.cuda.current_stream(logits.device).cuda_stream
        ws = get_workspace(lib.sv_sample_workspace_bytes(B, V, dt), logits.device, stream)
        self._keep = (logits, uniforms, greedy, ws)
        self._fn = lib.sv_sample
        self._args = (C.c_void_p(logits.data_ptr()), C.c_int32(dt), C.c_void_p(uniforms.data_ptr()),
                      C.c_float(float(temperature)), C.c_void_p(None if greedy is None else greedy.data_ptr()),
                      C.c_int32(B), C.c_int32(V), C.c_void_p(self.tokens.data_ptr()), None,
                      C.c_void_p(ws.data_ptr()), C.c_size_t(ws.numel()), C.c_void_p(stream))

    def __call__(self):
        _check_rc(self._fn(*self._args))
        return self.tokens


class BoundKvCommit:
    """sv_kv_commit on fixed tensors with pre-marshalled arguments."""

    def __init__(self, cache, cache_len, staged, accepted_len, offset=1, stream=None):
        torch = _torch()
        P, B, L = cache.shape[:3]
        row_bytes = cache[0, 0, 0].numel() * cache.element_size()
        K = staged.shape[2] - offset
        self.status = torch.empty(B, dtype=torch.int32, device=cache.device)
        if stream is None:
            stream = torch.cuda.current_stream(cache.device).cuda_stream
        self._keep = (cache, cache_len, staged, accepted_len)
        self._fn = load_library().sv_kv_commit
        self._args = (C.c_void_p(cache.data_ptr()), C.c_void_p(cache_len.data_ptr()), C.c_void_p(staged.data_ptr()),
                      C.c_void_p(accepted_len.data_ptr()), C.c_int32(P), C.c_int32(B), C.c_int32(K),
                      C.c_int32(offset), C.c_int64(L), C.c_int64(row_bytes), C.c_void_p(self.status.data_ptr()),
                      C.c_void_p(stream))

    def __call__(self):
        _check_rc(self._fn(*self._args))
        return self.status
