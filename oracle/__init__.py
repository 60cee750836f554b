"""fp64 CPU oracle for the speculative verify / logit-fusion pass.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The GPU library and
its Python binding never import this package, and this package imports
nothing from them.

The arithmetic lives in ``vwl_oracle.c`` (plain C, double precision, one row
at a time, plain sequential sums); this module builds it with gcc, loads it
with ctypes and marshals numpy arrays.  Each entry point follows the pages:

* ``asym`` -- AsymSpec reading notes, section 4.1 (context gain
  ``delta = a - b`` and the delta-fusion token ``argmax(t + beta*delta)``)
  and section 4.2 (``D = JSD(softmax(a) || softmax(b))``, the CDA threshold
  ``gamma*exp(-D)``, the acceptance test and emission at the first rejection);
  with the ablation variants of the same notes: ``delta = a`` or
  ``delta = t - b`` and the fixed threshold ``gamma`` without CDA.
* ``rapid`` -- RAPID notes, key design 2 (``zhat = z + eta*T*(q - p)``,
  ``phat = softmax(zhat/T)``), key design 3 (tail protection below 10% of the
  peak) and key design 4 (residual ``norm(max(p - phat, p - q, 0))``), with
  rejection sampling against the augmented target (overall framework).
* ``asym_lmhead`` -- the AsymSpec pass on logits produced from hidden states
  by the drafter's and the verifier's LM heads (fp64 library matmul, then
  ``asym``), with the error bound of an fp32 product-sum of the heads.
* ``asym_xfam`` -- the AsymSpec pass across model families (AsymSpec
  notes, analysis of cross-family pairs): the drafter's gain reaches the
  verifier through a vocabulary alignment, generation restricted to the
  paired tokens.
* ``e2sci`` -- E2-SCI notes, key design 3 (online adaptive verification:
  per-position JSD of drafter and target against the window's threshold,
  the EWMA credit state r = (1-beta) r + beta * accept_len/W, and the next
  threshold clamp(T_base + alpha*omega*(r - tau_credit), T_min, T_max)).
* ``rapid_zhat`` / ``rapid_phat`` -- the same definitions for one row, used
  by the pins.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against library routines (scipy), closed forms, the pages' bounds and
special cases, brute force and exact enumeration of the sampling law.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vwl_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

TAIL_EPS = 1e-6

_lib = None


def build(force: bool = True) -> str:
    """Compile ``vwl_oracle.c`` with gcc (OpenMP, no fast-math) into liboracle.so."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i = ctypes.c_int
    d = ctypes.c_double
    lib.vwl_oracle_asym.argtypes = [P, P, P, i, P, i, i, i, d, d, i, i, P, P, P, P, P, P, P, P, P, P, i]
    lib.vwl_oracle_asym.restype = i
    lib.vwl_oracle_rapid.argtypes = [P, P, i, P, P, P, i, i, i, d, d,
                                     P, P, P, P, P, P, P, P, P, P, P, d, P, P, i]
    lib.vwl_oracle_rapid.restype = i
    lib.vwl_oracle_rapid_zhat.argtypes = [P, P, i, d, d, P]
    lib.vwl_oracle_rapid_zhat.restype = i
    lib.vwl_oracle_rapid_phat.argtypes = [P, P, i, d, d, P]
    lib.vwl_oracle_rapid_phat.restype = i
    lib.vwl_oracle_asym_xfam.argtypes = [P, P, i, P, i, P, i, P, i, i, d, d, P, P, P, P, P, P, P, P, P, P, i]
    lib.vwl_oracle_asym_xfam.restype = i
    lib.vwl_oracle_e2sci.argtypes = [P, P, i, i, i, i, P, P, P, d, d, d, d, d, d, P, P, P, P, P, i]
    lib.vwl_oracle_e2sci.restype = i
    lib.vwl_oracle_max_threads.argtypes = []
    lib.vwl_oracle_max_threads.restype = i
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().vwl_oracle_max_threads())


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.c_void_p)


def _stored(x: np.ndarray, dtype: str) -> tuple[np.ndarray, int]:
    """Accept float32 values (widened by the oracle) or uint16 bf16 bits."""
    if dtype == "bf16":
        if x.dtype == np.uint16:
            return np.ascontiguousarray(x), 1
        x = np.ascontiguousarray(x, dtype=np.float32)
        bits = x.view(np.uint32)
        if np.any(bits & 0xFFFF):
            raise ValueError("bf16 workload holds values that are not bf16-exact")
        return np.ascontiguousarray((bits >> 16).astype(np.uint16)), 1
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32), 0
    raise ValueError(dtype)


DELTA_SOURCES = {"a-b": 0, "a": 1, "t-b": 2}
GATES = {"cda": 0, "fixed": 1}


@dataclass
class AsymResult:
    lse: np.ndarray        # [B, K+1, 3] log-sum-exp of a, b, t
    D: np.ndarray          # [B, K+1]
    gamma_eff: np.ndarray  # [B, K+1] the threshold in use (gamma under the fixed gate)
    fused: np.ndarray      # [B, K+1] int32
    gap: np.ndarray        # [B, K+1]
    top: np.ndarray        # [B, K+1] maximum fused score
    accept: np.ndarray     # [B, K] uint8
    margin: np.ndarray     # [B, K]
    accept_len: np.ndarray  # [B] int32
    token: np.ndarray      # [B] int32


def asym(a, b, t, draft, beta: float, gamma: float, dtype: str = "f32",
         nthreads: int = 0, delta: str = "a-b", gate: str = "cda") -> AsymResult:
    """Oracle of the AsymSpec verify pass on [B, K+1, V] rows.

    ``beta`` and ``gamma`` should be the float32 values the device receives
    (they are widened exactly).  ``delta`` picks the fusion source ("a-b",
    "a", "t-b") and ``gate`` the threshold ("cda" or "fixed")."""
    lib = _load()
    sa, dt = _stored(a, dtype)
    sb, _ = _stored(b, dtype)
    st, _ = _stored(t, dtype)
    B, P, V = sa.shape
    K = P - 1
    draft = np.ascontiguousarray(draft, dtype=np.int32).reshape(B, K)
    R = B * P
    lse = np.zeros((B, P, 3))
    D = np.zeros((B, P))
    ge = np.zeros((B, P))
    fused = np.zeros((B, P), np.int32)
    gap = np.zeros((B, P))
    top = np.zeros((B, P))
    acc = np.zeros((B, max(K, 0)), np.uint8)
    margin = np.zeros((B, max(K, 0)))
    alen = np.zeros(B, np.int32)
    tok = np.zeros(B, np.int32)
    rc = lib.vwl_oracle_asym(_ptr(sa), _ptr(sb), _ptr(st), dt, _ptr(draft), B, K, V,
                             float(np.float32(beta)), float(np.float32(gamma)),
                             DELTA_SOURCES[delta], GATES[gate], _ptr(lse), _ptr(D), _ptr(ge), _ptr(fused), _ptr(gap), _ptr(top),
                             _ptr(acc), _ptr(margin), _ptr(alen), _ptr(tok), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle asym failed with code %d" % rc)
    del R
    return AsymResult(lse, D, ge, fused, gap, top, acc, margin, alen, tok)


def asym_xfam(a, b, t, vmap, draft, beta: float, gamma: float, dtype: str = "f32",
              nthreads: int = 0) -> AsymResult:
    """Oracle of the cross-family AsymSpec pass: drafter rows a, b [B, K+1, Vd],
    verifier rows t [B, K+1, Vt], vmap [Vt] (drafter id paired with each
    verifier token, or -1), drafts [B, K] in verifier ids."""
    lib = _load()
    sa, dt = _stored(a, dtype)
    sb, _ = _stored(b, dtype)
    st, _ = _stored(t, dtype)
    B, P, Vd = sa.shape
    Vt = st.shape[2]
    if st.shape[:2] != (B, P) or sb.shape != sa.shape:
        raise ValueError("a, b must be [B, K+1, Vd] and t [B, K+1, Vt]")
    K = P - 1
    vmap = np.ascontiguousarray(vmap, dtype=np.int32).reshape(Vt)
    draft = np.ascontiguousarray(draft, dtype=np.int32).reshape(B, K)
    lse = np.zeros((B, P, 3))
    D = np.zeros((B, P))
    ge = np.zeros((B, P))
    fused = np.zeros((B, P), np.int32)
    gap = np.zeros((B, P))
    top = np.zeros((B, P))
    acc = np.zeros((B, max(K, 0)), np.uint8)
    margin = np.zeros((B, max(K, 0)))
    alen = np.zeros(B, np.int32)
    tok = np.zeros(B, np.int32)
    rc = lib.vwl_oracle_asym_xfam(_ptr(sa), _ptr(sb), Vd, _ptr(st), Vt, _ptr(vmap), dt, _ptr(draft), B, K,
                                  float(np.float32(beta)), float(np.float32(gamma)),
                                  _ptr(lse), _ptr(D), _ptr(ge), _ptr(fused), _ptr(gap), _ptr(top),
                                  _ptr(acc), _ptr(margin), _ptr(alen), _ptr(tok), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle asym_xfam failed with code %d" % rc)
    return AsymResult(lse, D, ge, fused, gap, top, acc, margin, alen, tok)


@dataclass
class LmheadResult:
    """The AsymSpec outputs on logits formed from hidden states and LM-head
    weights, with the per-logit bound on the error of any fp32 summation
    order of the H products (|h|.|W| * n * 2^-24 / (1 - n * 2^-24), n = H;
    zero where the inputs are dyadic enough that no partial sum rounds)."""
    res: AsymResult
    err_a: np.ndarray   # [B, K+1] largest bound over the row's a logits
    err_b: np.ndarray   # [B, K+1]
    err_t: np.ndarray   # [B, K+1]
    err_bd: np.ndarray  # [B, K] bound of b at the draft
    err_td: np.ndarray  # [B, K] bound of t at the draft


def _widen_bf16(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bits = np.ascontiguousarray(x, np.float32).view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("LM-head inputs must be bf16-exact")
    return x.astype(np.float64)


def asym_lmhead(h_a, h_b, W_d, h_t, W_t, draft, beta: float, gamma: float, delta: str = "a-b",
                gate: str = "cda", nthreads: int = 0) -> LmheadResult:
    """Oracle of AsymSpec on logits produced from hidden states by LM heads:
    a = h_a W_d^T, b = h_b W_d^T (the drafter's two views share its head),
    t = h_t W_t^T; h_* are [B, K+1, H] and W_* [V, H], all bf16 values.  The
    logits are formed in fp64 (a library matmul on the exactly widened
    inputs); the pass then follows asym()."""
    ha, hb, ht = (_widen_bf16(x) for x in (h_a, h_b, h_t))
    Wd, Wt = _widen_bf16(W_d), _widen_bf16(W_t)
    B, P, Hd = ha.shape
    V = Wd.shape[0]
    a = np.ascontiguousarray(ha.reshape(B * P, Hd) @ Wd.T).reshape(B, P, V)
    b = np.ascontiguousarray(hb.reshape(B * P, Hd) @ Wd.T).reshape(B, P, V)
    t = np.ascontiguousarray(ht.reshape(B * P, ht.shape[2]) @ Wt.T).reshape(B, P, V)
    lib = _load()
    K = P - 1
    draft = np.ascontiguousarray(draft, dtype=np.int32).reshape(B, K)
    lse = np.zeros((B, P, 3))
    D = np.zeros((B, P))
    ge = np.zeros((B, P))
    fused = np.zeros((B, P), np.int32)
    gap = np.zeros((B, P))
    top = np.zeros((B, P))
    acc = np.zeros((B, max(K, 0)), np.uint8)
    margin = np.zeros((B, max(K, 0)))
    alen = np.zeros(B, np.int32)
    tok = np.zeros(B, np.int32)
    rc = lib.vwl_oracle_asym(_ptr(a), _ptr(b), _ptr(t), 2, _ptr(draft), B, K, V,
                             float(np.float32(beta)), float(np.float32(gamma)),
                             DELTA_SOURCES[delta], GATES[gate], _ptr(lse), _ptr(D), _ptr(ge), _ptr(fused),
                             _ptr(gap), _ptr(top), _ptr(acc), _ptr(margin), _ptr(alen), _ptr(tok), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle asym (lm head) failed with code %d" % rc)
    res = AsymResult(lse, D, ge, fused, gap, top, acc, margin, alen, tok)
    u = 2.0 ** -24

    def lowest_bit(x):
        """Smallest power of two that divides every nonzero entry of the bf16
        array x, from its bit patterns (the implicit leading one included), or
        None if all entries are zero; 0.0 if any is infinite or NaN."""
        x = np.asarray(x)
        bits = x if x.dtype == np.uint16 else (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16)
        seen = np.flatnonzero(np.bincount(bits.astype(np.uint16).ravel(), minlength=65536))
        seen = seen[(seen & 0x7FFF) != 0]
        if seen.size == 0:
            return None
        e = (seen >> 7) & 0xFF
        if np.any(e == 0xFF):
            return 0.0
        sig = np.where(e == 0, seen & 0x7F, (seen & 0x7F) | 0x80).astype(np.int64)
        low = (sig & -sig).astype(np.float64)
        return float(np.min(np.ldexp(low, np.maximum(e, 1) - 127 - 7)))

    def bound(h, W, hs, Ws):
        """|h|.|W| * n u / (1 - n u), or 0 where the sum is exact in any order:
        every product of two bf16 values is exact in fp32, every product and
        every partial sum is an integer multiple of q = lowest_bit(h) *
        lowest_bit(W), and when q >= 2^-149 (no product underflows) and the
        absolute sum is at most 2^24 q (and finite in fp32) each such multiple
        is representable in fp32, so no product or addition rounds."""
        n = h.shape[-1]
        g = n * u / (1 - n * u)
        qh, qw = lowest_bit(hs), lowest_bit(Ws)
        if qh is None or qw is None:
            return np.zeros((B, P, W.shape[0]))
        q = qh * qw
        limit = min(2.0 ** 24 * q, float(np.finfo(np.float32).max)) if q >= 2.0 ** -149 else -1.0
        if n * float(np.max(np.abs(h))) * float(np.max(np.abs(W))) <= limit:
            return np.zeros((B, P, W.shape[0]))      # every sum is below the limit
        s = (np.abs(h.reshape(-1, n)) @ np.abs(W).T).reshape(B, P, -1)
        return np.where(s <= limit, 0.0, g * s)

    ea, eb, et = bound(ha, Wd, h_a, W_d), bound(hb, Wd, h_b, W_d), bound(ht, Wt, h_t, W_t)
    bi = np.arange(B)[:, None]
    ii = np.arange(K)[None, :]
    d = np.clip(draft, 0, V - 1)
    return LmheadResult(res, ea.max(axis=2), eb.max(axis=2), et.max(axis=2),
                        eb[bi, ii, d] if K else np.zeros((B, 0)), et[bi, ii, d] if K else np.zeros((B, 0)))


@dataclass
class E2sciParams:
    """Controller constants of the E2-SCI threshold update (key design 3);
    the pages fix only the EWMA decay (0.3), the rest are the caller's.
    The last four are the stabilisers the same passage names without a rule
    or constants (their reading is in e2sci_stabilise); their defaults
    switch them off."""
    alpha: float = 1.0
    tau_credit: float = 0.5
    T_base: float = 0.1
    T_min: float = 0.01
    T_max: float = 0.3
    ewma: float = 0.3
    hysteresis: float = 0.0   # dead band on the threshold change
    min_refresh: int = 1      # windows a threshold stays in effect at least
    delta: float = 0.0        # acceptance floor of the safety check
    T_safe: float = 0.0       # conservative threshold the safety check falls back to


@dataclass
class E2sciResult:
    D: np.ndarray           # [B, W]
    accept: np.ndarray      # [B, W] uint8
    accept_len: np.ndarray  # [B] int32
    r_hat: np.ndarray       # [B] updated smoothed acceptance
    T_next: np.ndarray      # [B] threshold of the next window (after the stabilisers)
    T_prop: np.ndarray = None       # [B] clamped proposal T_base + alpha*omega*(r - tau)
    age: np.ndarray = None          # [B] windows the next threshold has already been in effect
    hyst_margin: np.ndarray = None  # [B] |T_prop - T_in| - hysteresis where the dead band decided, else NaN


def e2sci_stabilise(T_in: float, T_prop: float, p_acc: float, age_in: int, prm: E2sciParams):
    """The E2-SCI stabilisers of one request after one window (key design 3
    names hysteresis, a minimum refresh interval and a hard safety check that
    falls back to a conservative threshold when Acc(T_pred) < delta; the page
    gives no rule or constant, so this is the plainest reading, applied in
    this order):
      1. safety check: the window's accepted fraction p_acc (accepted prefix
         length / W, measured at the predicted threshold T_in) below delta
         sets the next threshold to T_safe and restarts the interval;
      2. minimum refresh interval: a threshold stays in effect for at least
         min_refresh windows; age_in counts the windows it was in effect
         before this one, so a refresh is allowed once age_in + 1 >=
         min_refresh;
      3. hysteresis: a refresh adopts the clamped proposal T_prop only when
         it differs from T_in by more than the dead band.
    Returns (T_next, age_out, margin); age_out is 0 when the threshold was
    set anew (by 1 or 3) and age_in + 1 otherwise (saturating at 2^31 - 1);
    margin is |T_prop - T_in| - hysteresis where step 3 decided, else NaN.
    Arithmetic in float64 on the float32 inputs and constants."""
    f = lambda v: float(np.float32(v))
    T_in, T_prop, delta, h = float(T_in), float(T_prop), f(prm.delta), f(prm.hysteresis)
    nxt = min(int(age_in) + 1, 2 ** 31 - 1)
    if p_acc < delta:
        return f(prm.T_safe), 0, float("nan")
    if nxt < int(prm.min_refresh):
        return T_in, nxt, float("nan")
    margin = abs(T_prop - T_in) - h
    if margin > 0.0:
        return T_prop, 0, margin
    return T_in, nxt, margin


def e2sci(y, z, T, omega, r_hat, params: E2sciParams = E2sciParams(), dtype: str = "f32",
          nthreads: int = 0, age=None) -> E2sciResult:
    """Oracle of the E2-SCI adaptive JSD acceptance on [B, W, V] rows of
    drafter (y) and target (z) logits; T, omega, r_hat are [B] float32 (the
    values the device receives) and the constants are widened from float32.
    age ([B] int, default zeros) is the stabilisers' count of windows each
    request's threshold has been in effect; the next thresholds are the
    clamped proposals passed through e2sci_stabilise."""
    lib = _load()
    sy, dt = _stored(y, dtype)
    sz, _ = _stored(z, dtype)
    B, Wn, V = sy.shape
    T = np.ascontiguousarray(T, dtype=np.float32).reshape(B)
    omega = np.ascontiguousarray(omega, dtype=np.float32).reshape(B)
    r_hat = np.ascontiguousarray(r_hat, dtype=np.float32).reshape(B)
    f = lambda v: float(np.float32(v))
    D = np.zeros((B, Wn))
    acc = np.zeros((B, Wn), np.uint8)
    alen = np.zeros(B, np.int32)
    r_out = np.zeros(B)
    T_out = np.zeros(B)
    rc = lib.vwl_oracle_e2sci(_ptr(sy), _ptr(sz), dt, B, Wn, V, _ptr(T), _ptr(omega), _ptr(r_hat),
                              f(params.alpha), f(params.tau_credit), f(params.T_base), f(params.T_min),
                              f(params.T_max), f(params.ewma), _ptr(D), _ptr(acc), _ptr(alen),
                              _ptr(r_out), _ptr(T_out), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle e2sci failed with code %d" % rc)
    age = np.zeros(B, np.int64) if age is None else np.asarray(age, np.int64).reshape(B)
    T_next = np.zeros(B)
    age_out = np.zeros(B, np.int64)
    margin = np.full(B, np.nan)
    for bi in range(B):
        T_next[bi], age_out[bi], margin[bi] = e2sci_stabilise(T[bi], T_out[bi], alen[bi] / Wn, age[bi], params)
    return E2sciResult(D, acc, alen, r_out, T_next, T_out, age_out, margin)


@dataclass
class RapidResult:
    rowstat: np.ndarray     # [B, G+1, 4] L_z, L_y, Mhat, L_zhat
    phat_draft: np.ndarray  # [B, G]
    q_draft: np.ndarray     # [B, G]
    accept: np.ndarray      # [B, G] uint8
    acc_rel: np.ndarray     # [B, G]
    tail_d_dist: np.ndarray  # [B, G]
    accept_len: np.ndarray  # [B]
    token: np.ndarray       # [B]
    resid_S: np.ndarray     # [B] (-1: drawn from p)
    draw_slack: np.ndarray  # [B]
    tail_close: np.ndarray  # [B]
    emit_dist: np.ndarray | None  # [B, V]
    emit_scale: np.ndarray | None  # [B, V] p + max(phat, q) on the emitting row


def rapid(z, y, draft, u_accept, u_sample, eta: float, T: float, dtype: str = "f32",
          want_dist: bool = False, tail_eps: float = TAIL_EPS, nthreads: int = 0) -> RapidResult:
    """Oracle of the RAPID verify pass on [B, G+1, V] rows."""
    lib = _load()
    sz, dt = _stored(z, dtype)
    sy, _ = _stored(y, dtype)
    B, P, V = sz.shape
    G = P - 1
    draft = np.ascontiguousarray(draft, dtype=np.int32).reshape(B, G)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32).reshape(B, G)
    us = np.ascontiguousarray(u_sample, dtype=np.float32).reshape(B, P)
    rowstat = np.zeros((B, P, 4))
    phd = np.zeros((B, G))
    qd = np.zeros((B, G))
    acc = np.zeros((B, G), np.uint8)
    arel = np.zeros((B, G))
    tdd = np.zeros((B, G))
    alen = np.zeros(B, np.int32)
    tok = np.zeros(B, np.int32)
    rs = np.zeros(B)
    slack = np.zeros(B)
    close = np.zeros(B, np.int32)
    dist = np.zeros((B, V)) if want_dist else None
    scale = np.zeros((B, V)) if want_dist else None
    rc = lib.vwl_oracle_rapid(_ptr(sz), _ptr(sy), dt, _ptr(draft), _ptr(ua), _ptr(us),
                              B, G, V, float(np.float32(eta)), float(np.float32(T)),
                              _ptr(rowstat), _ptr(phd), _ptr(qd), _ptr(acc), _ptr(arel), _ptr(tdd),
                              _ptr(alen), _ptr(tok), _ptr(rs), _ptr(slack), _ptr(close),
                              float(tail_eps), _ptr(dist) if dist is not None else None,
                              _ptr(scale) if scale is not None else None, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle rapid failed with code %d" % rc)
    return RapidResult(rowstat, phd, qd, acc, arel, tdd, alen, tok, rs, slack, close, dist, scale)


def rapid_zhat(z: np.ndarray, y: np.ndarray, eta: float, T: float) -> np.ndarray:
    """zhat = z + eta*T*(softmax(y/T) - softmax(z/T)) for one row (float64)."""
    lib = _load()
    z = np.ascontiguousarray(z, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.zeros_like(z)
    if lib.vwl_oracle_rapid_zhat(_ptr(z), _ptr(y), z.size, float(eta), float(T), _ptr(out)):
        raise RuntimeError("oracle rapid_zhat failed")
    return out


def rapid_phat(z: np.ndarray, y: np.ndarray, eta: float, T: float) -> np.ndarray:
    """Tail-protected augmented target of one row (float64)."""
    lib = _load()
    z = np.ascontiguousarray(z, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.zeros_like(z)
    if lib.vwl_oracle_rapid_phat(_ptr(z), _ptr(y), z.size, float(eta), float(T), _ptr(out)):
        raise RuntimeError("oracle rapid_phat failed")
    return out
