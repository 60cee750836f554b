"""Seeded synthetic inputs for the speculative verify / logit-fusion pass.

This module is shared by the fp64 oracle side and the HIP side of every test,
by ``bench.py`` and by ``__graft_entry__.smoke``.  It draws random logits and
plants structure (displaced spikes, identical drafter rows, exact ties); it
holds none of the verification arithmetic itself: no softmax, no divergence,
no acceptance rule.  Random numbers that the method consumes (the RAPID
acceptance and residual uniforms) are drawn here and handed to both sides as
inputs.

Recipe (one logit row = one draft position of one request):

* ``z0 ~ N(0, 2^2)`` over the vocabulary and one spike index ``s``;
  ``z = z0`` with ``z[s] += 8``.
* AsymSpec: ``a = z + N(0, 0.5^2)``, ``t = z + N(0, 0.5^2)``; ``b = z +
  N(0, 0.5^2)`` except in an exact fraction of rows (seeded permutation) where
  the spike is removed from ``s`` and placed at ``s' != s`` before the noise is
  added.  Rows are produced in float64, rounded to float32 (round to nearest
  even) and, for bf16 workloads, rounded again to bf16 (round to nearest
  even).  Drafts are the drafter's greedy tokens ``d_i = argmax a_i`` (lowest
  index) on the stored values, for the first K positions of each request.
* "identical" rows set ``b := a`` bit for bit after rounding, so the context
  gain is exactly zero.
* "tie" rows get one column ``c`` that holds the row maxima of ``t`` and ``a``
  and the row minimum of ``b`` (values copied from the row, so nothing leaves
  the stored grid), and that whole column is then copied to a second index
  ``j``.  Any fused score that is non-decreasing in ``t`` and in ``a - b``
  (every ``t + beta*(a - b)`` with ``beta >= 0``) then has an exact tie at its
  maximum, and ``a`` has an exact tie at its maximum, whatever the evaluation
  order or precision.
* AsymSpec across families: drafter rows a, b over the drafter vocabulary
  Vd as in AsymSpec; a vocabulary alignment pairs ``n_shared`` verifier ids
  (a seeded random subset of the verifier vocabulary Vt, plus the last
  ``n_special`` ids of each vocabulary paired in order, standing in for
  special tokens) with distinct drafter ids (seeded random); the verifier row
  is ``t[v] = z[map[v]] + N(0, 0.5^2)`` on paired ids and ``N(0, 2^2)``
  elsewhere.  Drafts are the drafter's greedy tokens restricted to the
  paired drafter ids, given as the paired verifier ids.
* AsymSpec from hidden states (LM heads): drafter head W_d [V, Hd] ~
  N(0, (2/sqrt(Hd))^2) and hidden states h_a ~ N(0, 1), so the logits
  h_a W_d^T are N(0, 2^2); each row plants a spike of +8 at a token s by
  adding 8 w_s/|w_s|^2 (w_s = W_d[s]) to h_a; h_b = h_a + N(0, 0.25^2) (the
  compressed view, logit noise ~0.5), with the spike moved to another token
  in an exact 30% of rows.  The verifier head W_t = [W_d | W_x] (Ht = 2 Hd,
  W_x ~ N(0, (0.5/sqrt(Hd))^2)) and h_t = [h_b + N(0, 0.1^2) | N(0, 1)], so
  t ~ b + N(0, 0.5^2) (the verifier reads the compressed context).  Drafts
  are the planted tokens s.  Everything is rounded to bf16.
* LM heads with dyadic entries (the exact-product variant): every weight and
  hidden value is a signed power of two, W_d = +-1/8 and h = +-1/4 with
  random signs (logits N(0, 1.6^2)); the spike of +8 at s flips 128 of the
  coordinates where h and W_d[s] disagree in sign; h_b flips 64 random
  coordinates of h_a (logit noise 0.5) and, in an exact 30% of rows, undoes
  the spike's flips and plants it at s' instead; h_t = [h_b with 16 flips |
  +-1/4] and W_x = +-1/32.  Every product is a multiple of 2^-7 and every
  logit's absolute product-sum stays below 2^7, so an fp32 sum of the
  products is exact in any order.
* E2-SCI: target ``z_t = z + N(0, 0.5^2)``; drafter ``y = z + N(0,
  sigma^2)`` with ``sigma`` uniform on [0.1, 1.0] per row (a spread of
  divergences); "identical" rows set ``y := z_t`` bit for bit (divergence
  exactly 0).  The caller-owned controller state is drawn per request:
  threshold ``T`` uniform on [0.02, 0.2], weight ``omega`` on [0.5, 2],
  smoothed acceptance ``r_hat`` on [0, 1], each rounded to float32.
* RAPID: ``base = z``; target ``z_t = base + N(0, 0.5^2)``; drafter ``y =
  base + N(0, 1)`` except in an exact fraction of rows where the spike is
  displaced as above.  Drafts ``x_i`` are samples from the drafter's
  tempered softmax, drawn with the Gumbel-max construction (``argmax(y/T +
  G)``, ``G`` standard Gumbel) from a separate seeded stream.  Acceptance
  and residual uniforms are ``k * 2^-24`` with ``k`` uniform on
  ``[0, 2^24)``: exact in float32 and never 1.  The spiked RAPID variant
  raises the planted spike to +13, so that the target's mass concentrates on
  few tokens and the augmentation strength eta changes the accept/reject and
  residual decisions at the full vocabulary.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 7000

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# storage helpers (rounding and bit views; no method arithmetic)
# --------------------------------------------------------------------------
def round_to_bf16(x32: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bf16 value (ties to even).

    Returns float32 values that are exactly representable in bf16.
    Inputs must be finite.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-exact float32 values, as uint16 (the stored bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not bf16-exact")
    return (bits >> 16).astype(np.uint16)


def stored(x: np.ndarray, dtype: str) -> np.ndarray:
    """The array exactly as a device buffer stores it (float32 or uint16 bf16 bits)."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits(x)
    raise ValueError(dtype)


def _to_dtype(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return round_to_bf16(x32) if dtype == BF16 else x32


def uniforms_2p24(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms k * 2^-24, k ~ U{0, ..., 2^24 - 1}; exact in float32, < 1."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _choose_rows(rng: np.random.Generator, pool: np.ndarray, count: int) -> np.ndarray:
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.permutation(pool)[:count])


def _flip(h: np.ndarray, coords: np.ndarray) -> None:
    h[coords] = -h[coords]


def _plant(g: np.random.Generator, h: np.ndarray, w: np.ndarray, m: int) -> np.ndarray:
    """Flip m coordinates of h whose sign disagrees with w's (raising h.w by
    2 m |h_i w_i|); returns the flipped coordinates."""
    dis = np.flatnonzero(np.sign(h) != np.sign(w))
    c = g.choice(dis, size=min(m, dis.size), replace=False)
    _flip(h, c)
    return c


def _parallel_rows(R: int, V: int, nbuf: int, fn) -> None:
    """Run ``fn(r, scratch_buffers)`` for every row; rows are independent and
    seeded one by one, so the result does not depend on the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    nthreads = max(1, min(8, os.cpu_count() or 1, R))
    chunks = [range(i, R, nthreads) for i in range(nthreads)]

    def work(rows):
        bufs = [np.empty(V, np.float64) for _ in range(nbuf)]
        for r in rows:
            fn(r, bufs)

    if nthreads == 1:
        work(range(R))
        return
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(work, chunks))


# --------------------------------------------------------------------------
# AsymSpec inputs
# --------------------------------------------------------------------------
@dataclass
class AsymInputs:
    """Logit rows a (drafter, full context), b (drafter, compressed context),
    t (verifier), each [B, K+1, V] float32 holding values exact in ``dtype``;
    greedy drafts [B, K] int32; and the fusion strength / threshold."""

    a: np.ndarray
    b: np.ndarray
    t: np.ndarray
    draft: np.ndarray
    dtype: str
    beta: float
    gamma: float
    seed: int
    displaced: np.ndarray = field(default=None)   # bool [B, K+1]
    identical: np.ndarray = field(default=None)   # bool [B, K+1]
    tie: np.ndarray = field(default=None)         # bool [B, K+1]
    name: str = ""

    @property
    def B(self):
        return self.a.shape[0]

    @property
    def K(self):
        return self.a.shape[1] - 1

    @property
    def V(self):
        return self.a.shape[2]

    def stored(self, which: str) -> np.ndarray:
        return stored(getattr(self, which), self.dtype)

    def algorithmic_bytes(self) -> int:
        es = 2 if self.dtype == BF16 else 4
        return 3 * self.a.shape[0] * self.a.shape[1] * self.V * es


def gen_asym(B: int, K: int, V: int, dtype: str = F32, seed: int = SEED_BASE,
             displaced_frac: float = 0.3, identical_frac: float = 0.0,
             tie_frac: float = 0.0, beta: float = 1.0, gamma: float = 0.5,
             base_std: float = 2.0, spike: float = 8.0, noise_std: float = 0.5,
             name: str = "") -> AsymInputs:
    """Generate one AsymSpec workload following the module recipe."""
    if B < 1 or K < 0 or V < 1:
        raise ValueError("need B >= 1, K >= 0, V >= 1")
    R = B * (K + 1)
    ss = np.random.SeedSequence(seed)
    s_rows, s_sel, s_tie = ss.spawn(3)
    sel = np.random.default_rng(s_sel)

    all_rows = np.arange(R)
    n_ident = int(round(identical_frac * R))
    ident_rows = _choose_rows(sel, all_rows, n_ident)
    rest = np.setdiff1d(all_rows, ident_rows)
    n_tie = int(round(tie_frac * R))
    tie_rows = _choose_rows(sel, rest, min(n_tie, rest.size))
    n_disp = int(round(displaced_frac * R))
    disp_pool = rest if V > 1 else np.zeros(0, dtype=np.int64)
    disp_rows = _choose_rows(sel, disp_pool, min(n_disp, disp_pool.size))

    displaced = np.zeros(R, bool)
    displaced[disp_rows] = True
    identical = np.zeros(R, bool)
    identical[ident_rows] = True
    tie = np.zeros(R, bool)
    tie[tie_rows] = True

    a = np.empty((R, V), np.float32)
    b = np.empty((R, V), np.float32)
    t = np.empty((R, V), np.float32)
    row_seeds = s_rows.spawn(R)

    def make_row(r, bufs):
        z0, z, n, zb = bufs
        g = np.random.default_rng(row_seeds[r])
        g.standard_normal(out=z0)
        z0 *= base_std
        s = int(g.integers(0, V))
        np.copyto(z, z0)
        z[s] += spike
        g.standard_normal(out=n)
        n *= noise_std
        n += z
        a[r] = _to_dtype(n, dtype)
        g.standard_normal(out=n)
        n *= noise_std
        n += z
        t[r] = _to_dtype(n, dtype)
        if displaced[r]:
            s2 = int(g.integers(0, V - 1))
            s2 = s2 + 1 if s2 >= s else s2
            np.copyto(zb, z0)
            zb[s2] += spike
            src_b = zb
        else:
            src_b = z
        g.standard_normal(out=n)
        n *= noise_std
        n += src_b
        b[r] = _to_dtype(n, dtype)
        if identical[r]:
            b[r] = a[r]

    _parallel_rows(R, V, 4, make_row)

    gt = np.random.default_rng(s_tie)
    for r in tie_rows:
        if V < 2:
            continue
        c = int(gt.integers(0, V))
        j = int(gt.integers(0, V - 1))
        j = j + 1 if j >= c else j
        a[r, c] = a[r].max()
        t[r, c] = t[r].max()
        b[r, c] = b[r].min()
        a[r, j], b[r, j], t[r, j] = a[r, c], b[r, c], t[r, c]

    a = a.reshape(B, K + 1, V)
    b = b.reshape(B, K + 1, V)
    t = t.reshape(B, K + 1, V)
    draft = np.argmax(a[:, :K, :], axis=2).astype(np.int32) if K > 0 else np.zeros((B, 0), np.int32)
    return AsymInputs(a=a, b=b, t=t, draft=np.ascontiguousarray(draft), dtype=dtype,
                      beta=float(beta), gamma=float(gamma), seed=seed,
                      displaced=displaced.reshape(B, K + 1),
                      identical=identical.reshape(B, K + 1),
                      tie=tie.reshape(B, K + 1), name=name)


# --------------------------------------------------------------------------
# AsymSpec across model families
# --------------------------------------------------------------------------
@dataclass
class XfamInputs:
    """Drafter rows a, b [B, K+1, Vd], verifier rows t [B, K+1, Vt], the
    alignment vmap [Vt] int32 (paired drafter id or -1) and greedy drafts
    [B, K] in verifier ids."""

    a: np.ndarray
    b: np.ndarray
    t: np.ndarray
    vmap: np.ndarray
    draft: np.ndarray
    dtype: str
    beta: float
    gamma: float
    seed: int
    name: str = ""

    @property
    def B(self):
        return self.a.shape[0]

    @property
    def K(self):
        return self.a.shape[1] - 1

    @property
    def Vd(self):
        return self.a.shape[2]

    @property
    def Vt(self):
        return self.t.shape[2]

    def algorithmic_bytes(self) -> int:
        es = 2 if self.dtype == BF16 else 4
        rows = self.a.shape[0] * self.a.shape[1]
        return rows * (2 * self.Vd + self.Vt) * es + 4 * self.Vt


def gen_xfam(B: int, K: int, Vd: int, Vt: int, n_shared: int, dtype: str = F32, seed: int = SEED_BASE + 7,
             n_special: int = 16, displaced_frac: float = 0.3, beta: float = 1.0, gamma: float = 0.5,
             noise_std: float = 0.5, name: str = "") -> XfamInputs:
    """Generate one cross-family workload following the module recipe."""
    n_special = min(n_special, Vd, Vt)
    if n_shared + n_special > min(Vd, Vt):
        raise ValueError("more pairs than tokens")
    x = gen_asym(B, K, Vd, dtype, seed, displaced_frac=displaced_frac, beta=beta, gamma=gamma,
                 noise_std=noise_std)
    ss = np.random.SeedSequence(seed + 1)
    s_map, s_rows = ss.spawn(2)
    g = np.random.default_rng(s_map)
    vmap = np.full(Vt, -1, np.int32)
    vt_ids = g.permutation(Vt - n_special)[:n_shared]
    vd_ids = g.permutation(Vd - n_special)[:n_shared]
    vmap[vt_ids] = vd_ids
    vmap[Vt - n_special:] = np.arange(Vd - n_special, Vd, dtype=np.int32)
    paired = vmap >= 0
    R = B * (K + 1)
    z = x.t.reshape(R, Vd)          # the AsymSpec verifier row: z + noise on the drafter vocabulary
    t = np.empty((R, Vt), np.float32)
    row_seeds = s_rows.spawn(R)

    def make_row(r, bufs):
        (n,) = bufs
        gr = np.random.default_rng(row_seeds[r])
        gr.standard_normal(out=n)
        n *= 2.0
        n[paired] = z[r, vmap[paired]].astype(np.float64) + noise_std * gr.standard_normal(int(paired.sum()))
        t[r] = _to_dtype(n, dtype)

    _parallel_rows(R, Vt, 1, make_row)
    t = t.reshape(B, K + 1, Vt)
    # greedy drafts on the paired drafter ids, as verifier ids
    inv = np.full(Vd, -1, np.int64)
    inv[vmap[paired]] = np.flatnonzero(paired)
    pd = np.sort(vmap[paired])
    draft = np.zeros((B, K), np.int32)
    for bi in range(B):
        for i in range(K):
            row = x.a[bi, i, pd]
            draft[bi, i] = inv[pd[int(np.argmax(row))]]
    return XfamInputs(a=x.a, b=x.b, t=t, vmap=vmap, draft=draft, dtype=dtype, beta=float(beta),
                      gamma=float(gamma), seed=seed, name=name)


# --------------------------------------------------------------------------
# AsymSpec from hidden states and LM heads
# --------------------------------------------------------------------------
@dataclass
class LmheadInputs:
    """Hidden states h_a, h_b [B, K+1, Hd], h_t [B, K+1, Ht], heads W_d
    [V, Hd], W_t [V, Ht] (float32 arrays holding bf16 values), drafts [B, K]."""

    h_a: np.ndarray
    h_b: np.ndarray
    h_t: np.ndarray
    W_d: np.ndarray
    W_t: np.ndarray
    draft: np.ndarray
    beta: float
    gamma: float
    seed: int
    dtype: str = BF16
    name: str = ""

    @property
    def B(self):
        return self.h_a.shape[0]

    @property
    def K(self):
        return self.h_a.shape[1] - 1

    @property
    def V(self):
        return self.W_d.shape[0]

    @property
    def Hd(self):
        return self.W_d.shape[1]

    @property
    def Ht(self):
        return self.W_t.shape[1]

    def weight_bytes(self) -> int:
        return 2 * self.V * (self.Hd + self.Ht)


def gen_lmhead(B: int, K: int, V: int, Hd: int, seed: int = SEED_BASE + 8, displaced_frac: float = 0.3,
               beta: float = 1.0, gamma: float = 0.5, name: str = "") -> LmheadInputs:
    """Generate one LM-head workload following the module recipe (Ht = 2 Hd)."""
    if B < 1 or K < 0 or V < 2 or Hd < 1:
        raise ValueError("need B >= 1, K >= 0, V >= 2, Hd >= 1")
    R = B * (K + 1)
    ss = np.random.SeedSequence(seed)
    s_w, s_h, s_sel = ss.spawn(3)
    gw = np.random.default_rng(s_w)
    W_d = round_to_bf16((gw.standard_normal((V, Hd)) * (2.0 / np.sqrt(Hd))).astype(np.float32))
    W_x = round_to_bf16((gw.standard_normal((V, Hd)) * (0.5 / np.sqrt(Hd))).astype(np.float32))
    W_t = np.ascontiguousarray(np.concatenate([W_d, W_x], axis=1))
    sel = np.random.default_rng(s_sel)
    disp = np.zeros(R, bool)
    disp[_choose_rows(sel, np.arange(R), int(round(displaced_frac * R)))] = True
    gh = np.random.default_rng(s_h)
    h_a = np.empty((R, Hd), np.float32)
    h_b = np.empty((R, Hd), np.float32)
    h_t = np.empty((R, 2 * Hd), np.float32)
    spike = np.empty(R, np.int64)
    for r in range(R):
        s = int(gh.integers(0, V))
        w = W_d[s].astype(np.float64)
        base = gh.standard_normal(Hd)
        ha = base + 8.0 * w / np.dot(w, w)
        hb = ha + 0.25 * gh.standard_normal(Hd)
        if disp[r]:
            s2 = int(gh.integers(0, V - 1))
            s2 = s2 + 1 if s2 >= s else s2
            w2 = W_d[s2].astype(np.float64)
            hb = hb - 8.0 * w / np.dot(w, w) + 8.0 * w2 / np.dot(w2, w2)
        h_a[r] = round_to_bf16(ha.astype(np.float32))
        h_b[r] = round_to_bf16(hb.astype(np.float32))
        hc = h_b[r].astype(np.float64) + 0.1 * gh.standard_normal(Hd)
        h_t[r] = round_to_bf16(np.concatenate([hc, gh.standard_normal(Hd)]).astype(np.float32))
        spike[r] = s
    P = K + 1
    draft = spike.reshape(B, P)[:, :K].astype(np.int32)
    return LmheadInputs(h_a=h_a.reshape(B, P, Hd), h_b=h_b.reshape(B, P, Hd), h_t=h_t.reshape(B, P, 2 * Hd),
                        W_d=W_d, W_t=W_t, draft=np.ascontiguousarray(draft), beta=float(beta),
                        gamma=float(gamma), seed=seed, name=name)


# --------------------------------------------------------------------------
# E2-SCI inputs
# --------------------------------------------------------------------------
@dataclass
class E2sciInputs:
    """Drafter logits y and target logits z, each [B, W, V] float32 holding
    values exact in ``dtype`` (W draft positions of one window per
    request), and the caller-owned controller state per request."""

    y: np.ndarray
    z: np.ndarray
    T: np.ndarray       # [B] float32 threshold of this window
    omega: np.ndarray   # [B] float32 adaptive weight
    r_hat: np.ndarray   # [B] float32 smoothed acceptance before this window
    dtype: str
    seed: int
    identical: np.ndarray = field(default=None)  # bool [B, W]
    name: str = ""

    @property
    def B(self):
        return self.y.shape[0]

    @property
    def W(self):
        return self.y.shape[1]

    @property
    def V(self):
        return self.y.shape[2]

    def algorithmic_bytes(self) -> int:
        es = 2 if self.dtype == BF16 else 4
        return 2 * self.y.shape[0] * self.y.shape[1] * self.V * es


def gen_lmhead_dyadic(B: int, K: int, V: int, Hd: int, seed: int = SEED_BASE + 9,
                      displaced_frac: float = 0.3, beta: float = 1.0, gamma: float = 0.5,
                      name: str = "") -> LmheadInputs:
    """LM-head workload whose products are exact in fp32 (module recipe,
    the dyadic variant; Ht = 2 Hd)."""
    if B < 1 or K < 0 or V < 2 or Hd < 128:
        raise ValueError("need B >= 1, K >= 0, V >= 2, Hd >= 128")
    R = B * (K + 1)
    ss = np.random.SeedSequence(seed)
    s_w, s_h, s_sel = ss.spawn(3)
    gw = np.random.default_rng(s_w)

    def signs(shape, mag):
        return (gw.integers(0, 2, size=shape, dtype=np.int8).astype(np.float32) * 2 - 1) * np.float32(mag)

    W_d = signs((V, Hd), 0.125)
    W_t = np.ascontiguousarray(np.concatenate([W_d, signs((V, Hd), 1.0 / 32)], axis=1))
    sel = np.random.default_rng(s_sel)
    disp = np.zeros(R, bool)
    disp[_choose_rows(sel, np.arange(R), int(round(displaced_frac * R)))] = True
    gh = np.random.default_rng(s_h)
    h_a = np.empty((R, Hd), np.float32)
    h_b = np.empty((R, Hd), np.float32)
    h_t = np.empty((R, 2 * Hd), np.float32)
    spike = np.empty(R, np.int64)
    for r in range(R):
        s = int(gh.integers(0, V))
        h = (gh.integers(0, 2, size=Hd).astype(np.float32) * 2 - 1) * np.float32(0.25)
        planted = _plant(gh, h, W_d[s], 128)
        h_a[r] = h
        hb = h.copy()
        if disp[r]:
            s2 = int(gh.integers(0, V - 1))
            s2 = s2 + 1 if s2 >= s else s2
            _flip(hb, planted)
            _plant(gh, hb, W_d[s2], 128)
        _flip(hb, gh.choice(Hd, size=64, replace=False))
        h_b[r] = hb
        hc = hb.copy()
        _flip(hc, gh.choice(Hd, size=16, replace=False))
        h_t[r, :Hd] = hc
        h_t[r, Hd:] = (gh.integers(0, 2, size=Hd).astype(np.float32) * 2 - 1) * np.float32(0.25)
        spike[r] = s
    P = K + 1
    draft = spike.reshape(B, P)[:, :K].astype(np.int32)
    return LmheadInputs(h_a=h_a.reshape(B, P, Hd), h_b=h_b.reshape(B, P, Hd), h_t=h_t.reshape(B, P, 2 * Hd),
                        W_d=W_d, W_t=W_t, draft=np.ascontiguousarray(draft), beta=float(beta),
                        gamma=float(gamma), seed=seed, name=name)


def gen_e2sci(B: int, W: int, V: int, dtype: str = F32, seed: int = SEED_BASE + 5,
              identical_frac: float = 0.0, noise_lo: float = 0.1, noise_hi: float = 1.0,
              base_std: float = 2.0, spike: float = 8.0, target_std: float = 0.5,
              T_range=(0.02, 0.2), name: str = "") -> E2sciInputs:
    """Generate one E2-SCI workload following the module recipe."""
    if B < 1 or W < 1 or V < 1:
        raise ValueError("need B >= 1, W >= 1, V >= 1")
    R = B * W
    ss = np.random.SeedSequence(seed)
    s_rows, s_sel, s_state = ss.spawn(3)
    sel = np.random.default_rng(s_sel)
    ident_rows = _choose_rows(sel, np.arange(R), int(round(identical_frac * R)))
    identical = np.zeros(R, bool)
    identical[ident_rows] = True
    y = np.empty((R, V), np.float32)
    z = np.empty((R, V), np.float32)
    row_seeds = s_rows.spawn(R)

    def make_row(r, bufs):
        base, n = bufs
        g = np.random.default_rng(row_seeds[r])
        g.standard_normal(out=base)
        base *= base_std
        base[int(g.integers(0, V))] += spike
        sigma = g.uniform(noise_lo, noise_hi)
        g.standard_normal(out=n)
        n *= target_std
        n += base
        z[r] = _to_dtype(n, dtype)
        g.standard_normal(out=n)
        n *= sigma
        n += base
        y[r] = _to_dtype(n, dtype)
        if identical[r]:
            y[r] = z[r]

    _parallel_rows(R, V, 2, make_row)
    st = np.random.default_rng(s_state)
    T = st.uniform(T_range[0], T_range[1], size=B).astype(np.float32)
    omega = st.uniform(0.5, 2.0, size=B).astype(np.float32)
    r_hat = st.uniform(0.0, 1.0, size=B).astype(np.float32)
    return E2sciInputs(y=y.reshape(B, W, V), z=z.reshape(B, W, V), T=T, omega=omega, r_hat=r_hat,
                       dtype=dtype, seed=seed, identical=identical.reshape(B, W), name=name)


# --------------------------------------------------------------------------
# RAPID inputs
# --------------------------------------------------------------------------
@dataclass
class RapidInputs:
    """Target logits z and RAG-drafter logits y, each [B, G+1, V] float32
    holding values exact in ``dtype``; drafts [B, G] int32 sampled from the
    drafter; uniforms u_accept [B, G] and u_sample [B, G+1] float32."""

    z: np.ndarray
    y: np.ndarray
    draft: np.ndarray
    u_accept: np.ndarray
    u_sample: np.ndarray
    dtype: str
    eta: float
    T: float
    seed: int
    displaced: np.ndarray = field(default=None)
    name: str = ""

    @property
    def B(self):
        return self.z.shape[0]

    @property
    def G(self):
        return self.z.shape[1] - 1

    @property
    def V(self):
        return self.z.shape[2]

    def stored(self, which: str) -> np.ndarray:
        return stored(getattr(self, which), self.dtype)

    def algorithmic_bytes(self) -> int:
        es = 2 if self.dtype == BF16 else 4
        return 2 * self.z.shape[0] * self.z.shape[1] * self.V * es


def gen_rapid(B: int, G: int, V: int, dtype: str = F32, seed: int = SEED_BASE + 3,
              displaced_frac: float = 0.4, eta: float = 10.0, T: float = 1.0,
              base_std: float = 2.0, spike: float = 8.0, target_std: float = 0.5,
              drafter_std: float = 1.0, name: str = "") -> RapidInputs:
    """Generate one RAPID workload following the module recipe."""
    if B < 1 or G < 0 or V < 1:
        raise ValueError("need B >= 1, G >= 0, V >= 1")
    R = B * (G + 1)
    ss = np.random.SeedSequence(seed)
    s_rows, s_sel, s_draft, s_unif = ss.spawn(4)
    sel = np.random.default_rng(s_sel)
    n_disp = int(round(displaced_frac * R)) if V > 1 else 0
    disp_rows = _choose_rows(sel, np.arange(R), n_disp)
    displaced = np.zeros(R, bool)
    displaced[disp_rows] = True

    z = np.empty((R, V), np.float32)
    y = np.empty((R, V), np.float32)
    row_seeds = s_rows.spawn(R)

    def make_row(r, bufs):
        z0, base, n, yb = bufs
        g = np.random.default_rng(row_seeds[r])
        g.standard_normal(out=z0)
        z0 *= base_std
        s = int(g.integers(0, V))
        np.copyto(base, z0)
        base[s] += spike
        g.standard_normal(out=n)
        n *= target_std
        n += base
        z[r] = _to_dtype(n, dtype)
        if displaced[r]:
            s2 = int(g.integers(0, V - 1))
            s2 = s2 + 1 if s2 >= s else s2
            np.copyto(yb, z0)
            yb[s2] += spike
            src_y = yb
        else:
            src_y = base
        g.standard_normal(out=n)
        n *= drafter_std
        n += src_y
        y[r] = _to_dtype(n, dtype)

    _parallel_rows(R, V, 4, make_row)
    z = z.reshape(B, G + 1, V)
    y = y.reshape(B, G + 1, V)

    # Drafter sampling: Gumbel-max over the stored drafter logits.
    gd = np.random.default_rng(s_draft)
    draft = np.zeros((B, G), np.int32)
    for bi in range(B):
        for i in range(G):
            u = gd.random(V)
            u = np.where(u <= 0.0, np.finfo(np.float64).tiny, u)
            gumbel = -np.log(-np.log(u))
            draft[bi, i] = int(np.argmax(y[bi, i].astype(np.float64) / T + gumbel))
    gu = np.random.default_rng(s_unif)
    u_accept = uniforms_2p24(gu, (B, G))
    u_sample = uniforms_2p24(gu, (B, G + 1))
    return RapidInputs(z=z, y=y, draft=draft, u_accept=u_accept, u_sample=u_sample,
                       dtype=dtype, eta=float(eta), T=float(T), seed=seed,
                       displaced=displaced.reshape(B, G + 1), name=name)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------
VOCAB_QWEN3 = 151936     # vocabulary width of the drafter/verifier family in the AsymSpec setup
VOCAB_LLAMA31 = 128256   # vocabulary width of the RAPID target family

C2_BETAS = (0.0, 1.0, 2.0)
C2_GAMMAS = (0.4, 0.5, 0.7, 1.0)
C3_ETAS = (5.0, 10.0, 20.0)


def tiny_asym(seed: int = SEED_BASE + 0) -> AsymInputs:
    """B=4, K=2, V=1024, fp32; beta=1, gamma=0.5."""
    return gen_asym(4, 2, 1024, F32, seed, displaced_frac=0.3, beta=1.0, gamma=0.5,
                    name="asym_tiny_B4_K2_V1024_f32")


def single_asym(seed: int = SEED_BASE + 1) -> AsymInputs:
    """B=1, K=2, V=151936, fp32; beta=1, gamma=0.5."""
    return gen_asym(1, 2, VOCAB_QWEN3, F32, seed, displaced_frac=0.3, beta=1.0, gamma=0.5,
                    name="asym_single_B1_K2_V151936_f32")


def batched_asym(seed: int = SEED_BASE + 2, beta: float = 1.0, gamma: float = 0.5) -> AsymInputs:
    """B=64, K=2, V=151936, bf16; the (beta, gamma) grid is swept on these inputs."""
    return gen_asym(64, 2, VOCAB_QWEN3, BF16, seed, displaced_frac=0.3, beta=beta,
                    gamma=gamma, name="asym_batched_B64_K2_V151936_bf16")


def rapid_c3(seed: int = SEED_BASE + 3, eta: float = 10.0) -> RapidInputs:
    """B=16, G=10, V=128256, fp32, T=1; eta in {5, 10, 20}."""
    return gen_rapid(16, 10, VOCAB_LLAMA31, F32, seed, displaced_frac=0.4, eta=eta, T=1.0,
                     name="rapid_B16_G10_V128256_f32")


def rapid_spiked(seed: int = SEED_BASE + 60, eta: float = 10.0) -> RapidInputs:
    """B=16, G=10, V=128256, fp32, T=1, spike +13: eta changes decisions."""
    return gen_rapid(16, 10, VOCAB_LLAMA31, F32, seed, displaced_frac=0.4, eta=eta, T=1.0, spike=13.0,
                     name="rapid_spiked_B16_G10_V128256_f32")


def large_asym(seed: int = SEED_BASE + 4, beta: float = 1.0, gamma: float = 0.5) -> AsymInputs:
    """B=256, K=4, V=151936, bf16; 20% identical drafter rows, 5% planted ties."""
    return gen_asym(256, 4, VOCAB_QWEN3, BF16, seed, displaced_frac=0.3,
                    identical_frac=0.2, tie_frac=0.05, beta=beta, gamma=gamma,
                    name="asym_large_B256_K4_V151936_bf16")


def e2sci_single(seed: int = SEED_BASE + 5) -> E2sciInputs:
    """B=1 (the pages' real-time batch), W=8 drafts, V=151936, bf16."""
    return gen_e2sci(1, 8, VOCAB_QWEN3, BF16, seed, identical_frac=0.25,
                     name="e2sci_B1_W8_V151936_bf16")


def e2sci_batched(seed: int = SEED_BASE + 6) -> E2sciInputs:
    """B=64 requests, W=8 drafts, V=151936, bf16."""
    return gen_e2sci(64, 8, VOCAB_QWEN3, BF16, seed, identical_frac=0.1,
                     name="e2sci_B64_W8_V151936_bf16")


VOCAB_SHARED_QWEN_LLAMA = 109566  # string-identical tokens of the page's alignment


def xfam_batched(seed: int = SEED_BASE + 7) -> XfamInputs:
    """B=64, K=2, Qwen-family drafter (Vd=151936), Llama-family verifier
    (Vt=128256), 109,566 shared tokens plus 16 special pairs, bf16."""
    return gen_xfam(64, 2, VOCAB_QWEN3, VOCAB_LLAMA31, VOCAB_SHARED_QWEN_LLAMA, BF16, seed,
                    name="xfam_B64_K2_Vd151936_Vt128256_bf16")


HIDDEN_QWEN3_4B = 2560   # the pages' main drafter (model card hidden size)


def lmhead_batched(seed: int = SEED_BASE + 8) -> LmheadInputs:
    """B=64, K=2, V=151936, Hd=2560 (Qwen3-4B drafter head), Ht=5120 (a
    Qwen3-32B-sized verifier head), bf16."""
    return gen_lmhead(64, 2, VOCAB_QWEN3, HIDDEN_QWEN3_4B, seed, name="lmhead_B64_K2_V151936_Hd2560_Ht5120_bf16")


def lmhead_dyadic(seed: int = SEED_BASE + 9) -> LmheadInputs:
    """The LM-head bench shape (B=64, K=2, V=151936, Hd=2560, Ht=5120) with
    signed power-of-two entries, so the logits are exact in fp32."""
    return gen_lmhead_dyadic(64, 2, VOCAB_QWEN3, HIDDEN_QWEN3_4B, seed,
                             name="lmhead_dyadic_B64_K2_V151936_Hd2560_Ht5120_bf16")
