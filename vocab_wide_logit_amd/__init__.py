"""Speculative verification and logit fusion over vocabulary-wide logit rows,
on AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``lib/libvwl.so`` (HIP kernels behind a C ABI,
declared in ``include/vwl.h``).  This module only marshals arguments:
it checks tensor placement and layout, allocates output tensors and a
zero-filled workspace with torch, passes raw device pointers and torch's
current HIP stream, and raises on a non-OK status.  Every step of the pass
runs in the library's kernels; there is no other implementation to fall
back to, and importing fails loudly when the library has not been built.

Entry points (same names as the C ABI):

* ``asym_verify`` -- AsymSpec verification (AsymSpec reading notes, sections
  4.1-4.2): JSD of the two drafter views, CDA threshold gamma*exp(-D),
  acceptance test, first-rejection scan, delta-fusion token.
* ``asym_verify_variant`` -- the same pass with the fusion source and the
  gate of the AsymSpec notes' mechanism ablation: delta = a - b, a or t - b;
  the CDA threshold or a fixed gamma.
* ``asym_verify_xfam`` -- the AsymSpec pass across model families: drafter
  rows on the drafter vocabulary, verifier rows on the verifier's, joined by
  a vocabulary alignment (verifier id -> paired drafter id or -1).
* ``asym_verify_lmhead`` -- the AsymSpec pass from hidden states: the LM
  heads' products on the matrix cores with the row statistics in their
  epilogue; the JSD from stored (a, b) pairs, or, with ``store_pairs=False``,
  from a and b formed a second time (no logit written).
* ``e2sci_verify`` -- E2-SCI adaptive JSD acceptance (E2-SCI notes, key
  design 3): per-position divergence of drafter and target against the
  window threshold, then the caller-owned credit state and next threshold.
* ``rapid_verify`` -- RAPID verification (RAPID notes, key designs 2-4):
  augmented target with tail protection, rejection test against it, and the
  adjusted residual draw from caller-supplied uniforms.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import NamedTuple, Optional

import torch  # loaded first so the library binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libvwl.so")

VWL_F32 = 0
VWL_BF16 = 1
DEVERR_DRAFT = 1
DEVERR_UNIFORM = 2
DEVERR_TIMEOUT = 4
DEVERR_MAP = 8
MAX_K = 63

_lib = None
_lib_lock = threading.Lock()

DELTA_SOURCES = {"a-b": 0, "a": 1, "t-b": 2}  # vwl_delta_source
GATES = {"cda": 0, "fixed": 1}                 # vwl_gate

SYMBOLS = ("vwl_status_string", "vwl_version", "vwl_workspace_reset",
           "vwl_asym_workspace_bytes", "asym_verify", "asym_verify_variant", "vwl_asym_plan_info",
           "vwl_rapid_workspace_bytes", "rapid_verify",
           "vwl_plan_info", "vwl_asym_check", "vwl_rapid_check",
           "vwl_set_plan_override", "vwl_set_xfam_override", "vwl_set_phase_event",
           "vwl_e2sci_workspace_bytes", "e2sci_verify", "vwl_e2sci_plan_info",
           "vwl_asym_xfam_workspace_bytes", "asym_verify_xfam",
           "vwl_asym_lmhead_workspace_bytes", "vwl_asym_lmhead_workspace_min_bytes", "asym_verify_lmhead",
           "asym_verify_noalloc")


class E2sciParams(ctypes.Structure):
    """vwl_e2sci_params: constants of the E2-SCI threshold update.  The page
    prints only the EWMA decay (0.3); the defaults of the others are this
    binding's choice."""
    _fields_ = [("alpha", ctypes.c_float), ("tau_credit", ctypes.c_float), ("T_base", ctypes.c_float),
                ("T_min", ctypes.c_float), ("T_max", ctypes.c_float), ("ewma", ctypes.c_float),
                ("hysteresis", ctypes.c_float), ("min_refresh", ctypes.c_int32), ("delta", ctypes.c_float),
                ("T_safe", ctypes.c_float)]

    def __init__(self, alpha=1.0, tau_credit=0.5, T_base=0.1, T_min=0.01, T_max=0.3, ewma=0.3,
                 hysteresis=0.0, min_refresh=1, delta=0.0, T_safe=0.0):
        super().__init__(alpha, tau_credit, T_base, T_min, T_max, ewma, hysteresis, min_refresh, delta, T_safe)


class VwlError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvwl.so and declare its signatures; raises if it is not built."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError("libvwl.so is not built (%s); run __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        f = ctypes.c_float
        sz = ctypes.c_size_t
        lib.vwl_status_string.argtypes = [i]
        lib.vwl_status_string.restype = ctypes.c_char_p
        lib.vwl_version.argtypes = []
        lib.vwl_version.restype = i
        lib.vwl_workspace_reset.argtypes = [P, sz, P]
        lib.vwl_workspace_reset.restype = i
        lib.vwl_asym_workspace_bytes.argtypes = [i, i, i, i]
        lib.vwl_asym_workspace_bytes.restype = sz
        lib.vwl_rapid_workspace_bytes.argtypes = [i, i, i, i]
        lib.vwl_rapid_workspace_bytes.restype = sz
        lib.asym_verify.argtypes = [P, P, P, P, i, i, i, i, f, f, P, P, P, P, P, P, P, P, sz, P]
        lib.asym_verify.restype = i
        lib.asym_verify_noalloc.argtypes = [P, P, P, P, i, i, i, i, f, f, P, P, P, P, P, P, P, P]
        lib.asym_verify_noalloc.restype = i
        lib.asym_verify_variant.argtypes = [P, P, P, P, i, i, i, i, f, f, i, i, P, P, P, P, P, P, P, P, sz, P]
        lib.asym_verify_variant.restype = i
        lib.vwl_asym_plan_info.argtypes = [i, i, i, i, i, i, ctypes.POINTER(ctypes.c_int64)]
        lib.vwl_asym_plan_info.restype = i
        lib.rapid_verify.argtypes = [P, P, P, P, P, i, i, i, i, f, f, P, P, P, P, P, P, P, P, sz, P]
        lib.rapid_verify.restype = i
        lib.vwl_plan_info.argtypes = [i, i, i, i, i, ctypes.POINTER(ctypes.c_int64)]
        lib.vwl_plan_info.restype = i
        lib.vwl_asym_check.argtypes = [P, P, P, P, i, i, i, i, f, f, P, P, P, P, P, P, P, sz, sz]
        lib.vwl_asym_check.restype = i
        lib.vwl_rapid_check.argtypes = [P, P, P, P, P, i, i, i, i, f, f, P, P, P, P, sz, sz]
        lib.vwl_rapid_check.restype = i
        lib.vwl_set_plan_override.argtypes = [i, i, i]
        lib.vwl_set_plan_override.restype = i
        lib.vwl_set_xfam_override.argtypes = [i, i]
        lib.vwl_set_xfam_override.restype = i
        lib.vwl_asym_lmhead_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.vwl_asym_lmhead_workspace_bytes.restype = sz
        lib.vwl_asym_lmhead_workspace_min_bytes.argtypes = [i, i, i, i, i]
        lib.vwl_asym_lmhead_workspace_min_bytes.restype = sz
        lib.asym_verify_lmhead.argtypes = [P, P, P, P, P, P, i, i, i, i, i, f, f, P, P, P, P, P, P, P, P, sz, P]
        lib.asym_verify_lmhead.restype = i
        lib.vwl_asym_xfam_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.vwl_asym_xfam_workspace_bytes.restype = sz
        lib.asym_verify_xfam.argtypes = [P, P, i, P, i, P, P, i, i, i, f, f, P, P, P, P, P, P, P, P, sz, P]
        lib.asym_verify_xfam.restype = i
        lib.vwl_e2sci_workspace_bytes.argtypes = [i, i, i, i]
        lib.vwl_e2sci_workspace_bytes.restype = sz
        lib.e2sci_verify.argtypes = [P, P, i, i, i, i, P, P, P, P, ctypes.POINTER(E2sciParams),
                                     P, P, P, P, P, P, sz, P]
        lib.e2sci_verify.restype = i
        lib.vwl_e2sci_plan_info.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_int64)]
        lib.vwl_e2sci_plan_info.restype = i
        lib.vwl_set_phase_event.argtypes = [P]
        lib.vwl_set_phase_event.restype = i
        _lib = lib
        return lib


def _check(code: int) -> None:
    if code != 0:
        msg = load_library().vwl_status_string(code).decode()
        raise VwlError(code, msg)


class PreparedCall:
    """A library call whose arguments were checked and marshalled once (from
    ``asym_verify``, ``e2sci_verify`` or ``rapid_verify`` with
    ``prepare=True``).  Each ``()`` issues the same C call again on the
    stream that was current at preparation, with the same input, output and
    workspace memory (the caller refills the inputs in place), and returns
    the output tuple.  It keeps those tensors alive.  For serving loops in
    which the host's per-call checks would dominate a small call's latency."""
    __slots__ = ("_fn", "_args", "_keep", "out")

    def __init__(self, fn, args, keep, out):
        self._fn, self._args, self._keep, self.out = fn, args, keep, out

    def __call__(self):
        code = self._fn(*self._args)
        if code:
            _check(code)
        return self.out


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return VWL_F32
    if x.dtype == torch.bfloat16:
        return VWL_BF16
    raise TypeError("logits must be float32 or bfloat16, got %s" % x.dtype)


def _ptr(x: Optional[torch.Tensor]):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _dev_tensor(x: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if dtype is not None and x.dtype != dtype:
        raise TypeError("%s must have dtype %s" % (name, dtype))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return x


# Workspace cache: one zero-filled buffer per (device, stream, mode, shape).
# The kernels leave it ready for the next call after every completed call.
# A call that ends with the timeout bit (VWL_DEVERR_TIMEOUT, 4) in dev_err
# leaves its workspace undefined: the caller drops the cached buffers with
# drop_workspaces() (or passes a fresh workspace) before the next call.  The
# binding does not look at dev_err itself, since reading it waits for the
# device.
_ws_cache: dict = {}
_ws_lock = threading.Lock()

VWL_DEVERR_DRAFT = 1
VWL_DEVERR_UNIFORM = 2
VWL_DEVERR_TIMEOUT = 4
VWL_DEVERR_MAP = 8


def drop_workspaces() -> int:
    """Forget every cached workspace (the next calls allocate zero-filled
    ones); returns how many were dropped.  Needed after a call whose dev_err
    has the timeout bit, whose workspace is then undefined."""
    with _ws_lock:
        n = len(_ws_cache)
        _ws_cache.clear()
    return n


def check_dev_err(dev_err: torch.Tensor) -> int:
    """Read a call's dev_err (waits for the device), drop the cached
    workspaces when it carries the timeout bit, and return its value."""
    v = int(dev_err.reshape(-1)[0].item())
    if v & VWL_DEVERR_TIMEOUT:
        drop_workspaces()
    return v


def _stream_ptr(device) -> int:
    """Raw handle of the current stream of `device` (the cheap query when
    this torch build has it: a call's host overhead bounds small calls)."""
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _workspace(mode: int, B: int, K: int, V: int, dt: int, device, stream: int) -> torch.Tensor:
    def need():
        lib = load_library()
        return (lib.vwl_asym_workspace_bytes if mode == 0 else lib.vwl_rapid_workspace_bytes)(B, K, V, dt)
    return _workspace_sized((mode, B, K, V, dt), need, device, stream)


def _workspace_sized(shape_key, need, device, stream: int) -> torch.Tensor:
    """The cached workspace of (device, stream, shape); `need()` gives its
    size in bytes and is asked only when none is cached."""
    key = (device.index, stream) + tuple(shape_key)
    ws = _ws_cache.get(key)
    if ws is not None:
        return ws
    n = int(need())
    if n == 0:
        _check(2)
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None:
            ws = torch.zeros(n, dtype=torch.uint8, device=device)
            _ws_cache[key] = ws
        return ws


def workspace_bytes(mode: str, B: int, K: int, V: int, dtype: torch.dtype) -> int:
    """Size of the workspace of one call ("asym" or "rapid")."""
    lib = load_library()
    dt = VWL_BF16 if dtype == torch.bfloat16 else VWL_F32
    f = lib.vwl_asym_workspace_bytes if mode == "asym" else lib.vwl_rapid_workspace_bytes
    return int(f(B, K, V, dt))


def plan_info(mode: str, B: int, K: int, V: int, dtype: torch.dtype) -> dict:
    """Launch plan the library picks on the current device."""
    lib = load_library()
    out = (ctypes.c_int64 * 6)()
    dt = VWL_BF16 if dtype == torch.bfloat16 else VWL_F32
    _check(lib.vwl_plan_info(0 if mode == "asym" else 1, B, K, V, dt, out))
    return {"team": out[0], "vec_per_thread": out[1], "teams": out[2], "grid": out[3],
            "threads": out[4], "rows": out[5]}


def asym_plan_info(B: int, K: int, V: int, dtype: torch.dtype, delta: str = "a-b", gate: str = "cda") -> dict:
    """Launch plan of one AsymSpec variant on the current device."""
    lib = load_library()
    out = (ctypes.c_int64 * 6)()
    dt = VWL_BF16 if dtype == torch.bfloat16 else VWL_F32
    _check(lib.vwl_asym_plan_info(B, K, V, dt, DELTA_SOURCES[delta], GATES[gate], out))
    return {"team": out[0], "vec_per_thread": out[1], "teams": out[2], "grid": out[3],
            "threads": out[4], "rows": out[5]}


def set_plan_override(mode: str, vec_per_thread: int = 0, max_teams: int = 0) -> None:
    """Tuning hook: pin vectors per thread / cap teams (0 = automatic)."""
    _check(load_library().vwl_set_plan_override(0 if mode == "asym" else 1, vec_per_thread, max_teams))


def set_xfam_override(general: bool = False, segs: int = 0) -> None:
    """Test/tuning hook of asym_verify_xfam: force the general verifier pass,
    or pin the staged pass's drafter segments per row (0 = automatic)."""
    _check(load_library().vwl_set_xfam_override(1 if general else 0, segs))


def set_phase_event(event) -> None:
    """Profiling hook: record ``event`` (a torch.cuda.Event, or None to stop)
    on the call's stream between the row kernel and the kernels after it."""
    ptr = None
    if event is not None:
        if not event.cuda_event:
            raise ValueError("record the event once before handing it to the library")
        ptr = ctypes.c_void_p(event.cuda_event)
    _check(load_library().vwl_set_phase_event(ptr))


class AsymOut(NamedTuple):
    D: torch.Tensor           # [B, K+1] float32
    gamma_eff: torch.Tensor   # [B, K+1] float32
    accept: torch.Tensor      # [B, K] uint8
    fused: torch.Tensor       # [B, K+1] int32
    accept_len: torch.Tensor  # [B] int32
    token: torch.Tensor       # [B] int32
    dev_err: torch.Tensor     # [1] int32


def asym_out(B: int, K: int, device) -> AsymOut:
    """Preallocated outputs for ``asym_verify(..., out=...)``."""
    kw = dict(device=device)
    return AsymOut(torch.empty(B, K + 1, dtype=torch.float32, **kw),
                   torch.empty(B, K + 1, dtype=torch.float32, **kw),
                   torch.empty(B, K, dtype=torch.uint8, **kw),
                   torch.empty(B, K + 1, dtype=torch.int32, **kw),
                   torch.empty(B, dtype=torch.int32, **kw),
                   torch.empty(B, dtype=torch.int32, **kw),
                   torch.zeros(1, dtype=torch.int32, **kw))


def asym_verify(a: torch.Tensor, b: torch.Tensor, t: torch.Tensor, draft: torch.Tensor,
                beta: float, gamma: float, *, out: Optional[AsymOut] = None,
                workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """AsymSpec verification of [B, K+1, V] logit rows on the current stream.

    a: drafter logits on the full context; b: drafter logits on the
    compressed context; t: verifier logits; draft: [B, K] int32 draft ids.
    Returns D, gamma_eff, accept, fused, accept_len, token and dev_err; with
    prepare=True, a PreparedCall that issues this call (nothing runs yet)."""
    lib = load_library()
    _dev_tensor(a, "a")
    dt = _dt(a)
    _dev_tensor(b, "b", a.dtype)
    _dev_tensor(t, "t", a.dtype)
    if a.dim() != 3 or b.shape != a.shape or t.shape != a.shape:
        raise ValueError("a, b, t must share one [B, K+1, V] shape")
    B, P, V = a.shape
    K = P - 1
    _dev_tensor(draft, "draft", torch.int32)
    if tuple(draft.shape) != (B, K):
        raise ValueError("draft must be [B, K]")
    if out is None:
        out = asym_out(B, K, a.device)
    stream = _stream_ptr(a.device)
    ws = workspace if workspace is not None else _workspace(0, B, K, V, dt, a.device, stream)
    args = (_ptr(a), _ptr(b), _ptr(t), _ptr(draft) if K > 0 else None,
            B, K, V, dt, float(beta), float(gamma),
            _ptr(out.D), _ptr(out.gamma_eff), _ptr(out.accept) if K > 0 else None,
            _ptr(out.fused), _ptr(out.accept_len), _ptr(out.token), _ptr(out.dev_err),
            _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    if prepare:
        return PreparedCall(lib.asym_verify, args, (a, b, t, draft, ws), out)
    _check(lib.asym_verify(*args))
    return out


def asym_verify_noalloc(a: torch.Tensor, b: torch.Tensor, t: torch.Tensor, draft: torch.Tensor,
                        beta: float, gamma: float, *, out: Optional[AsymOut] = None) -> AsymOut:
    """``asym_verify`` through the library's no-allocation entry point: the
    workspace is the library's static per-device scratch (16 MiB), so the
    call itself allocates nothing once ``out`` is given.  Calls that may
    overlap on one device share that scratch and must be ordered."""
    lib = load_library()
    _dev_tensor(a, "a")
    dt = _dt(a)
    _dev_tensor(b, "b", a.dtype)
    _dev_tensor(t, "t", a.dtype)
    if a.dim() != 3 or b.shape != a.shape or t.shape != a.shape:
        raise ValueError("a, b, t must share one [B, K+1, V] shape")
    B, P, V = a.shape
    K = P - 1
    _dev_tensor(draft, "draft", torch.int32)
    if tuple(draft.shape) != (B, K):
        raise ValueError("draft must be [B, K]")
    if out is None:
        out = asym_out(B, K, a.device)
    stream = _stream_ptr(a.device)
    code = lib.asym_verify_noalloc(_ptr(a), _ptr(b), _ptr(t), _ptr(draft) if K > 0 else None,
                                   B, K, V, dt, float(beta), float(gamma),
                                   _ptr(out.D), _ptr(out.gamma_eff), _ptr(out.accept) if K > 0 else None,
                                   _ptr(out.fused), _ptr(out.accept_len), _ptr(out.token), _ptr(out.dev_err),
                                   ctypes.c_void_p(stream))
    _check(code)
    return out


def asym_verify_variant(a: Optional[torch.Tensor], b: torch.Tensor, t: torch.Tensor, draft: torch.Tensor,
                        beta: float, gamma: float, delta: str = "a-b", gate: str = "cda", *,
                        out: Optional[AsymOut] = None, workspace: Optional[torch.Tensor] = None) -> AsymOut:
    """AsymSpec verification with fusion source ``delta`` ("a-b", "a", "t-b")
    and threshold ``gate`` ("cda": gamma*exp(-D); "fixed": gamma, D not
    computed and returned as NaN).  ``a`` may be None only for
    delta="t-b" with gate="fixed", the one variant that never reads it."""
    lib = load_library()
    if delta not in DELTA_SOURCES or gate not in GATES:
        raise ValueError("delta must be one of %s and gate one of %s" % (list(DELTA_SOURCES), list(GATES)))
    _dev_tensor(t, "t")
    dt = _dt(t)
    _dev_tensor(b, "b", t.dtype)
    if a is not None:
        _dev_tensor(a, "a", t.dtype)
        if a.shape != t.shape:
            raise ValueError("a, b, t must share one [B, K+1, V] shape")
    elif not (delta == "t-b" and gate == "fixed"):
        raise ValueError("a is required unless delta='t-b' and gate='fixed'")
    if t.dim() != 3 or b.shape != t.shape:
        raise ValueError("a, b, t must share one [B, K+1, V] shape")
    B, P, V = t.shape
    K = P - 1
    _dev_tensor(draft, "draft", torch.int32)
    if tuple(draft.shape) != (B, K):
        raise ValueError("draft must be [B, K]")
    if out is None:
        out = asym_out(B, K, t.device)
    stream = _stream_ptr(t.device)
    ws = workspace if workspace is not None else _workspace(0, B, K, V, dt, t.device, stream)
    code = lib.asym_verify_variant(_ptr(a), _ptr(b), _ptr(t), _ptr(draft) if K > 0 else None,
                                   B, K, V, dt, float(beta), float(gamma), DELTA_SOURCES[delta], GATES[gate],
                                   _ptr(out.D), _ptr(out.gamma_eff), _ptr(out.accept) if K > 0 else None,
                                   _ptr(out.fused), _ptr(out.accept_len), _ptr(out.token), _ptr(out.dev_err),
                                   _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    _check(code)
    return out


def asym_verify_xfam(a: torch.Tensor, b: torch.Tensor, t: torch.Tensor, vmap: torch.Tensor,
                     draft: torch.Tensor, beta: float, gamma: float, *, out: Optional[AsymOut] = None,
                     workspace: Optional[torch.Tensor] = None) -> AsymOut:
    """AsymSpec across model families on the current stream.  a, b: drafter
    logits [B, K+1, Vd]; t: verifier logits [B, K+1, Vt]; vmap: [Vt] int32
    (paired drafter id or -1); draft: [B, K] int32 verifier ids."""
    lib = load_library()
    _dev_tensor(a, "a")
    dt = _dt(a)
    _dev_tensor(b, "b", a.dtype)
    _dev_tensor(t, "t", a.dtype)
    if a.dim() != 3 or b.shape != a.shape or t.dim() != 3 or t.shape[:2] != a.shape[:2]:
        raise ValueError("a, b must be [B, K+1, Vd] and t [B, K+1, Vt]")
    B, P, Vd = a.shape
    Vt = t.shape[2]
    K = P - 1
    _dev_tensor(vmap, "vmap", torch.int32)
    if tuple(vmap.shape) != (Vt,):
        raise ValueError("vmap must be [Vt]")
    _dev_tensor(draft, "draft", torch.int32)
    if tuple(draft.shape) != (B, K):
        raise ValueError("draft must be [B, K]")
    if out is None:
        out = asym_out(B, K, a.device)
    stream = _stream_ptr(a.device)
    if workspace is None:
        workspace = _workspace_sized(("xfam", B, K, Vd, Vt, dt),
                                     lambda: lib.vwl_asym_xfam_workspace_bytes(B, K, Vd, Vt, dt), a.device, stream)
    code = lib.asym_verify_xfam(_ptr(a), _ptr(b), Vd, _ptr(t), Vt, _ptr(vmap), _ptr(draft) if K > 0 else None,
                                B, K, dt, float(beta), float(gamma),
                                _ptr(out.D), _ptr(out.gamma_eff), _ptr(out.accept) if K > 0 else None,
                                _ptr(out.fused), _ptr(out.accept_len), _ptr(out.token), _ptr(out.dev_err),
                                _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
    _check(code)
    return out


def asym_verify_lmhead(h_a: torch.Tensor, h_b: torch.Tensor, W_d: torch.Tensor, h_t: torch.Tensor,
                       W_t: torch.Tensor, draft: torch.Tensor, beta: float, gamma: float, *,
                       out: Optional[AsymOut] = None, workspace: Optional[torch.Tensor] = None,
                       store_pairs: bool = True) -> AsymOut:
    """AsymSpec from hidden states on the current stream (bf16 tensors):
    h_a, h_b [B, K+1, Hd], h_t [B, K+1, Ht], W_d [V, Hd], W_t [V, Ht];
    draft [B, K] int32.  store_pairs: the cached workspace holds the fp32
    (a, b) pairs (8 B (K+1) V bytes) for the JSD pass; False sizes it for
    the path that forms a and b twice instead.  A caller's workspace picks
    the path by its size."""
    lib = load_library()
    for name, x in (("h_a", h_a), ("h_b", h_b), ("W_d", W_d), ("h_t", h_t), ("W_t", W_t)):
        _dev_tensor(x, name, torch.bfloat16)
    if h_a.dim() != 3 or h_b.shape != h_a.shape or h_t.dim() != 3 or h_t.shape[:2] != h_a.shape[:2]:
        raise ValueError("h_a, h_b must be [B, K+1, Hd] and h_t [B, K+1, Ht]")
    B, P, Hd = h_a.shape
    Ht = h_t.shape[2]
    V = W_d.shape[0]
    if tuple(W_d.shape) != (V, Hd) or tuple(W_t.shape) != (V, Ht):
        raise ValueError("W_d must be [V, Hd] and W_t [V, Ht]")
    K = P - 1
    _dev_tensor(draft, "draft", torch.int32)
    if tuple(draft.shape) != (B, K):
        raise ValueError("draft must be [B, K]")
    if out is None:
        out = asym_out(B, K, h_a.device)
    stream = _stream_ptr(h_a.device)
    if workspace is None:
        size = lib.vwl_asym_lmhead_workspace_bytes if store_pairs else lib.vwl_asym_lmhead_workspace_min_bytes
        workspace = _workspace_sized(("lmhead", bool(store_pairs), B, K, V, Hd, Ht),
                                     lambda: size(B, K, V, Hd, Ht), h_a.device, stream)
    code = lib.asym_verify_lmhead(_ptr(h_a), _ptr(h_b), _ptr(W_d), _ptr(h_t), _ptr(W_t),
                                  _ptr(draft) if K > 0 else None, B, K, V, Hd, Ht, float(beta), float(gamma),
                                  _ptr(out.D), _ptr(out.gamma_eff), _ptr(out.accept) if K > 0 else None,
                                  _ptr(out.fused), _ptr(out.accept_len), _ptr(out.token), _ptr(out.dev_err),
                                  _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
    _check(code)
    return out


class E2sciOut(NamedTuple):
    D: torch.Tensor           # [B, W] float32
    accept: torch.Tensor      # [B, W] uint8
    accept_len: torch.Tensor  # [B] int32
    T_next: torch.Tensor      # [B] float32 threshold of the next window
    r_hat: torch.Tensor       # [B] float32 credit state (updated in place)
    dev_err: torch.Tensor     # [1] int32
    age: Optional[torch.Tensor] = None  # [B] int32 stabiliser window count (updated in place), if given


def e2sci_plan_info(B: int, W: int, V: int, dtype: torch.dtype) -> dict:
    lib = load_library()
    out = (ctypes.c_int64 * 6)()
    dt = VWL_BF16 if dtype == torch.bfloat16 else VWL_F32
    _check(lib.vwl_e2sci_plan_info(B, W, V, dt, out))
    return {"team": out[0], "vec_per_thread": out[1], "teams": out[2], "grid": out[3],
            "threads": out[4], "rows": out[5]}


class E2sciBuffers(NamedTuple):
    """Preallocated per-call outputs of ``e2sci_verify(..., out=...)``."""
    D: torch.Tensor           # [B, W] float32
    accept: torch.Tensor      # [B, W] uint8
    accept_len: torch.Tensor  # [B] int32
    dev_err: torch.Tensor     # [1] int32, bits OR-ed in across calls


def e2sci_out(B: int, W: int, device) -> E2sciBuffers:
    """Preallocated outputs for ``e2sci_verify(..., out=...)``."""
    kw = dict(device=device)
    return E2sciBuffers(torch.empty(B, W, dtype=torch.float32, **kw), torch.empty(B, W, dtype=torch.uint8, **kw),
                        torch.empty(B, dtype=torch.int32, **kw), torch.zeros(1, dtype=torch.int32, **kw))


def e2sci_verify(y: torch.Tensor, z: torch.Tensor, T: torch.Tensor, omega: torch.Tensor,
                 r_hat: torch.Tensor, params: Optional[E2sciParams] = None, *,
                 age: Optional[torch.Tensor] = None,
                 T_out: Optional[torch.Tensor] = None, out: Optional[E2sciBuffers] = None,
                 workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """E2-SCI adaptive JSD acceptance of one window per request on the
    current stream.  y: drafter logits, z: target logits, [B, W, V];
    T, omega, r_hat: [B] float32 device tensors (r_hat is updated in place);
    age: [B] int32 device tensor of the stabilisers' window count, updated in
    place (needed when params.min_refresh > 1); the next thresholds go to
    T_out (a new tensor when None; pass T itself to update in place).  With
    ``out`` (from ``e2sci_out``) the call allocates nothing once the
    workspace is cached; its dev_err keeps the bits of earlier calls.  With
    prepare=True, returns a PreparedCall that issues this call."""
    lib = load_library()
    _dev_tensor(y, "y")
    dt = _dt(y)
    _dev_tensor(z, "z", y.dtype)
    if y.dim() != 3 or z.shape != y.shape:
        raise ValueError("y and z must share one [B, W, V] shape")
    B, Wn, V = y.shape
    for name, x in (("T", T), ("omega", omega), ("r_hat", r_hat)):
        _dev_tensor(x, name, torch.float32)
        if tuple(x.shape) != (B,):
            raise ValueError("%s must be [B]" % name)
    if T_out is None:
        T_out = torch.empty(B, dtype=torch.float32, device=y.device)
    _dev_tensor(T_out, "T_out", torch.float32)
    if age is not None:
        _dev_tensor(age, "age", torch.int32)
        if tuple(age.shape) != (B,):
            raise ValueError("age must be [B]")
    params = params if params is not None else E2sciParams()
    if out is None:
        out = e2sci_out(B, Wn, y.device)
    else:
        for name, x, shape, dtype in (("D", out.D, (B, Wn), torch.float32), ("accept", out.accept, (B, Wn), torch.uint8),
                                      ("accept_len", out.accept_len, (B,), torch.int32),
                                      ("dev_err", out.dev_err, (1,), torch.int32)):
            _dev_tensor(x, "out." + name, dtype)
            if tuple(x.shape) != shape:
                raise ValueError("out.%s must be %s" % (name, list(shape)))
    D, acc, alen, err = out
    stream = _stream_ptr(y.device)
    if workspace is None:
        workspace = _workspace_sized(("e2sci", B, Wn, V, dt),
                                     lambda: lib.vwl_e2sci_workspace_bytes(B, Wn, V, dt), y.device, stream)
    args = (_ptr(y), _ptr(z), B, Wn, V, dt, _ptr(T), _ptr(omega), _ptr(r_hat),
            _ptr(age) if age is not None else None, ctypes.byref(params), _ptr(D), _ptr(acc), _ptr(alen),
            _ptr(T_out), _ptr(err), _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
    result = E2sciOut(D, acc, alen, T_out, r_hat, err, age)
    if prepare:
        return PreparedCall(lib.e2sci_verify, args, (y, z, T, omega, r_hat, age, params, T_out, workspace), result)
    _check(lib.e2sci_verify(*args))
    return result


class RapidOut(NamedTuple):
    accept: torch.Tensor       # [B, G] uint8
    accept_len: torch.Tensor   # [B] int32
    token: torch.Tensor        # [B] int32
    p_hat_draft: Optional[torch.Tensor]  # [B, G] float32
    q_draft: Optional[torch.Tensor]      # [B, G] float32
    emit_dist: Optional[torch.Tensor]    # [B, V] float32
    dev_err: torch.Tensor      # [1] int32


def rapid_out(B: int, G: int, V: int, device, want_probs: bool = False,
              want_dist: bool = False) -> RapidOut:
    """Preallocated outputs for ``rapid_verify(..., out=...)``."""
    kw = dict(device=device)
    return RapidOut(torch.empty(B, G, dtype=torch.uint8, **kw),
                    torch.empty(B, dtype=torch.int32, **kw),
                    torch.empty(B, dtype=torch.int32, **kw),
                    torch.empty(B, G, dtype=torch.float32, **kw) if want_probs else None,
                    torch.empty(B, G, dtype=torch.float32, **kw) if want_probs else None,
                    torch.empty(B, V, dtype=torch.float32, **kw) if want_dist else None,
                    torch.zeros(1, dtype=torch.int32, **kw))


def rapid_verify(z: torch.Tensor, y: torch.Tensor, draft: torch.Tensor,
                 u_accept: torch.Tensor, u_sample: torch.Tensor, eta: float, T: float,
                 *, want_probs: bool = False, want_dist: bool = False,
                 out: Optional[RapidOut] = None,
                 workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """RAPID verification of [B, G+1, V] logit rows on the current stream.

    z: target logits; y: RAG-drafter logits; draft: [B, G] int32;
    u_accept: [B, G] and u_sample: [B, G+1] float32 uniforms in [0, 1).
    With prepare=True, returns a PreparedCall that issues this call."""
    lib = load_library()
    _dev_tensor(z, "z")
    dt = _dt(z)
    _dev_tensor(y, "y", z.dtype)
    if z.dim() != 3 or y.shape != z.shape:
        raise ValueError("z, y must share one [B, G+1, V] shape")
    B, P, V = z.shape
    G = P - 1
    _dev_tensor(draft, "draft", torch.int32)
    _dev_tensor(u_accept, "u_accept", torch.float32)
    _dev_tensor(u_sample, "u_sample", torch.float32)
    if tuple(draft.shape) != (B, G) or tuple(u_accept.shape) != (B, G) or tuple(u_sample.shape) != (B, P):
        raise ValueError("draft, u_accept must be [B, G] and u_sample [B, G+1]")
    if out is None:
        out = rapid_out(B, G, V, z.device, want_probs, want_dist)
    stream = _stream_ptr(z.device)
    ws = workspace if workspace is not None else _workspace(1, B, G, V, dt, z.device, stream)
    args = (_ptr(z), _ptr(y), _ptr(draft) if G > 0 else None,
            _ptr(u_accept) if G > 0 else None, _ptr(u_sample),
            B, G, V, dt, float(eta), float(T),
            _ptr(out.accept) if G > 0 else None, _ptr(out.accept_len), _ptr(out.token),
            _ptr(out.p_hat_draft), _ptr(out.q_draft), _ptr(out.emit_dist),
            _ptr(out.dev_err), _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    if prepare:
        return PreparedCall(lib.rapid_verify, args, (z, y, draft, u_accept, u_sample, ws), out)
    _check(lib.rapid_verify(*args))
    return out


def to_device_logits(x_f32, dtype: str, device="cuda") -> torch.Tensor:
    """Move float32 host values (exact in ``dtype``) to a device tensor of that dtype."""
    t = torch.from_numpy(x_f32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: the values are bf16-representable
    return t.to(device).contiguous()
