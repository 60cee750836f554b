"""Pins of the fp64 oracle to things other than itself.

Each test ties one oracle output to an independent library routine (scipy),
a closed form, a bound or special case stated on the pages, brute force on
tiny inputs, or exact enumeration of a sampling law.  Chosen so that a dropped
term, a wrong sign, a wrong index or a transposed operand in the oracle fails
at least one of them.

Citations: "AsymSpec notes 4.1/4.2/4.4" = the AsymSpec reading notes page,
sections 4.1 (delta-fusion), 4.2 (CDA gate), 4.4 (engineering); "RAPID
notes design N" = the RAPID notes page, key design N.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.spatial.distance import jensenshannon
from scipy.special import log_softmax, logsumexp, softmax

import oracle
import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
LN2 = math.log(2.0)


def _rows(B, K, V, seed, scale=2.0, dyadic=False):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, scale, size=(3, B, K + 1, V))
    if dyadic:  # multiples of 2^-10: shifts by small integers stay exact
        x = np.round(x * 1024) / 1024
    x = x.astype(np.float32)
    draft = rng.integers(0, V, size=(B, K)).astype(np.int32)
    return x[0], x[1], x[2], draft


def _asym(a, b, t, draft, beta=1.0, gamma=0.5, dtype="f32"):
    return oracle.asym(a, b, t, draft, beta, gamma, dtype)


# ---------------------------------------------------------------- softmax / LSE
@pytest.mark.parametrize("V", [1, 2, 3, 17, 1024])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lse_matches_scipy(oracle_lib, V, dtype):
    """Row log-sum-exp (the softmax normaliser of AsymSpec notes 4.2) against scipy."""
    a, b, t, d = _rows(2, 2, V, 11 + V)
    if dtype == "bf16":
        a, b, t = (W.round_to_bf16(x) for x in (a, b, t))
    r = _asym(a, b, t, d, dtype=dtype)
    for j, x in enumerate((a, b, t)):
        ref = logsumexp(x.astype(np.float64), axis=2)
        np.testing.assert_allclose(r.lse[..., j], ref, rtol=1e-13, atol=1e-13)


def test_shift_invariance(oracle_lib):
    """Adding a constant to a row leaves its softmax unchanged: D, the fused
    token, the test and the scan are unchanged, the normaliser moves by c."""
    a, b, t, d = _rows(3, 2, 64, 5, dyadic=True)
    r0 = _asym(a, b, t, d)
    for c in (3.0, -5.0):
        r1 = _asym(a + np.float32(c), b + np.float32(c), t + np.float32(c), d)
        np.testing.assert_allclose(r1.D, r0.D, rtol=1e-9, atol=1e-15)
        np.testing.assert_array_equal(r1.fused, r0.fused)
        np.testing.assert_array_equal(r1.accept, r0.accept)
        np.testing.assert_array_equal(r1.accept_len, r0.accept_len)
        np.testing.assert_allclose(r1.lse, r0.lse + c, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- JSD
@pytest.mark.parametrize("V", [2, 5, 1024, 20000])
def test_jsd_matches_scipy(oracle_lib, V):
    """D = JSD(softmax(a) || softmax(b)) (AsymSpec notes 4.2) against scipy's
    Jensen-Shannon distance squared (natural log)."""
    a, b, t, d = _rows(2, 1, V, 100 + V)
    r = _asym(a, b, t, d)
    for bi in range(2):
        for i in range(2):
            p = softmax(a[bi, i].astype(np.float64))
            q = softmax(b[bi, i].astype(np.float64))
            ref = jensenshannon(p, q) ** 2
            assert r.D[bi, i] == pytest.approx(ref, rel=1e-9, abs=1e-15)


def test_jsd_two_token_closed_form(oracle_lib):
    """V=2: JSD = H(m) - (H(p)+H(q))/2 with binary entropies in nats."""
    def H(x):
        return -(x * math.log(x) + (1 - x) * math.log(1 - x))
    for xa, xb in [(0.3, -1.2), (2.0, 2.0), (-4.0, 3.5), (0.0, 0.25)]:
        a = np.array([[[xa, 0.0]]], np.float32)
        b = np.array([[[xb, 0.0]]], np.float32)
        r = _asym(a, b, a, np.zeros((1, 0), np.int32))
        pa = 1 / (1 + math.exp(-float(np.float32(xa))))
        pb = 1 / (1 + math.exp(-float(np.float32(xb))))
        ref = H(0.5 * (pa + pb)) - 0.5 * (H(pa) + H(pb))
        assert r.D[0, 0] == pytest.approx(ref, rel=1e-12, abs=1e-16)


def test_identical_rows_give_zero_gain(oracle_lib):
    """a == b: delta = 0 (AsymSpec notes 4.1), so D = 0 exactly, gamma_eff =
    gamma exactly, and the fused token is argmax t (lowest index)."""
    a, _, t, d = _rows(4, 2, 300, 9)
    r = _asym(a, a.copy(), t, d, beta=1.7, gamma=0.45)
    assert np.all(r.D == 0.0)
    assert np.all(r.gamma_eff == np.float64(np.float32(0.45)))
    np.testing.assert_array_equal(r.fused, np.argmax(t, axis=2))


def test_disjoint_spikes_reach_ln2(oracle_lib):
    """Distributions with disjoint support reach the ln 2 bound (AsymSpec notes 4.2)."""
    V = 8
    a = np.zeros((1, 1, V), np.float32)
    b = np.zeros((1, 1, V), np.float32)
    a[0, 0, 1] = 1000.0
    b[0, 0, 6] = 1000.0
    r = _asym(a, b, a, np.zeros((1, 0), np.int32), gamma=0.5)
    assert r.D[0, 0] == pytest.approx(LN2, abs=1e-12)
    assert r.gamma_eff[0, 0] == pytest.approx(0.25, abs=1e-12)


def test_bounds_on_workloads(oracle_lib):
    """JSD in [0, ln 2] hence gamma_eff in [gamma/2, gamma] (AsymSpec notes 4.2)."""
    ub = GOLDEN["jsd_upper_bound"]["value"]
    lo, hi = GOLDEN["gamma_eff_range"]["value"]
    x = W.tiny_asym()
    r = _asym(x.a, x.b, x.t, x.draft, x.beta, x.gamma)
    g = float(np.float32(x.gamma))
    assert np.all(r.D >= 0) and np.all(r.D <= ub)
    assert np.all(r.gamma_eff >= lo * g - 1e-15) and np.all(r.gamma_eff <= hi * g + 1e-15)


# ---------------------------------------------------------------- fused token
def test_fused_steering_sign(oracle_lib):
    """delta-fusion argmax(t + beta*(a - b)) (AsymSpec notes 4.1): a context
    gain at index 1 moves the token there for beta > 0; beta = 0 keeps argmax t
    with the lowest index on the tie."""
    t = np.array([[[1.0, 1.0, 0.0]]], np.float32)
    a = np.array([[[0.0, 2.0, 0.0]]], np.float32)
    b = np.array([[[0.0, 0.0, 0.0]]], np.float32)
    nod = np.zeros((1, 0), np.int32)
    assert _asym(a, b, t, nod, beta=1.0).fused[0, 0] == 1
    assert _asym(a, b, t, nod, beta=0.0).fused[0, 0] == 0
    # the gain is a - b, not b - a: the same column in b pushes away
    assert _asym(b, a, t, nod, beta=1.0).fused[0, 0] == 0
    # strong negative gain at index 0 moves the token to index 1
    a2 = np.array([[[-3.0, 0.0, 0.0]]], np.float32)
    assert _asym(a2, b, t, nod, beta=0.5).fused[0, 0] == 1
    # beta weights the gain: t favours 2 by 1.0, gain favours 0 by 0.75
    t3 = np.array([[[0.0, 0.0, 1.0]]], np.float32)
    a3 = np.array([[[0.75, 0.0, 0.0]]], np.float32)
    assert _asym(a3, b, t3, nod, beta=1.0).fused[0, 0] == 2
    assert _asym(a3, b, t3, nod, beta=2.0).fused[0, 0] == 0


@pytest.mark.parametrize("V", [1, 2, 3, 5, 8])
def test_fused_brute_force_tiny(oracle_lib, V):
    """Exhaustive check of the lowest-index argmax on small integer grids,
    where ties are frequent."""
    rng = np.random.default_rng(V)
    for _ in range(40):
        a = rng.integers(-2, 3, size=(1, 1, V)).astype(np.float32)
        b = rng.integers(-2, 3, size=(1, 1, V)).astype(np.float32)
        t = rng.integers(-2, 3, size=(1, 1, V)).astype(np.float32)
        beta = float(rng.integers(0, 3))
        r = _asym(a, b, t, np.zeros((1, 0), np.int32), beta=beta)
        f = int(r.fused[0, 0])
        score = [float(t[0, 0, v]) + beta * (float(a[0, 0, v]) - float(b[0, 0, v])) for v in range(V)]
        best = max(score)
        assert score[f] == best
        assert all(score[v] < best for v in range(f))
        n_best = sum(s == best for s in score)
        assert (r.gap[0, 0] == 0.0) == (n_best > 1) or V == 1


def test_planted_ties(oracle_lib):
    """Tie rows of the workload generator: exact tie at the fused maximum for
    every beta >= 0, and the lowest of the tied indices is chosen."""
    x = W.gen_asym(8, 2, 512, "bf16", seed=77, tie_frac=0.5, identical_frac=0.0)
    rows = np.argwhere(x.tie)
    assert len(rows) == 12
    for beta in (0.0, 1.0, 2.0):
        r = _asym(x.a, x.b, x.t, x.draft, beta=beta, dtype="bf16")
        for bi, i in rows:
            score = x.t[bi, i].astype(np.float64) + beta * (x.a[bi, i].astype(np.float64) - x.b[bi, i])
            tied = np.flatnonzero(score == score.max())
            assert len(tied) >= 2
            assert r.gap[bi, i] == 0.0
            assert r.fused[bi, i] == tied.min()


# ---------------------------------------------------------------- acceptance test
def test_accept_closed_form_two_tokens(oracle_lib):
    """Test of AsymSpec notes 4.2 on V=2 rows, where softmax is the logistic
    function: accept iff sigma(x_t) > gamma*exp(-D)*sigma(x_b)."""
    cases = [(1.0, 0.5, 0.0, 0.5), (0.0, 1.0, 1.0, 0.5), (0.0, 1.0, 1.0, 0.9),
             (-1.0, 1.0, -0.5, 0.2), (2.0, -3.0, 0.5, 1.0)]
    for xt, xb, xa, g in cases:
        t = np.array([[[xt, 0.0], [0.0, 0.0]]], np.float32)
        b = np.array([[[xb, 0.0], [0.0, 0.0]]], np.float32)
        a = np.array([[[xa, 0.0], [0.0, 0.0]]], np.float32)
        d = np.array([[0]], np.int32)
        r = _asym(a, b, t, d, beta=1.0, gamma=g)
        sig = lambda v: 1 / (1 + math.exp(-float(np.float32(v))))
        pa, pb = sig(xa), sig(xb)
        H = lambda x: -(x * math.log(x) + (1 - x) * math.log(1 - x))
        D = H(0.5 * (pa + pb)) - 0.5 * (H(pa) + H(pb))
        gf = float(np.float32(g))
        expect = sig(xt) > gf * math.exp(-D) * pb
        assert bool(r.accept[0, 0]) == expect
        margin = math.log(sig(xt)) - math.log(pb) - math.log(gf) + D
        assert r.margin[0, 0] == pytest.approx(margin, abs=1e-12)


def test_accept_margin_matches_scipy(oracle_lib):
    """The log-space margin of the test, rebuilt from scipy's log_softmax and
    Jensen-Shannon distance, and the flag agrees with its sign."""
    a, b, t, d = _rows(5, 3, 700, 42)
    g = 0.55
    r = _asym(a, b, t, d, beta=0.7, gamma=g)
    gf = float(np.float32(g))
    for bi in range(5):
        for i in range(3):
            D = jensenshannon(softmax(a[bi, i].astype(np.float64)), softmax(b[bi, i].astype(np.float64))) ** 2
            lt = log_softmax(t[bi, i].astype(np.float64))[d[bi, i]]
            lb = log_softmax(b[bi, i].astype(np.float64))[d[bi, i]]
            m = lt - lb - math.log(gf) + D
            assert r.margin[bi, i] == pytest.approx(m, abs=1e-9)
            assert bool(r.accept[bi, i]) == (m > 0)


def test_accept_is_strict(oracle_lib):
    """The printed test is a strict inequality (AsymSpec notes 4.2): with
    a = b = t and gamma = 1, D = 0 and p_t(d) equals gamma_eff * p_b(d)
    exactly, which rejects."""
    a, _, _, d = _rows(3, 2, 50, 77)
    r = _asym(a, a.copy(), a.copy(), d, beta=1.0, gamma=1.0)
    assert np.all(r.D == 0.0)
    assert np.all(r.accept == 0) and np.all(r.accept_len == 0)
    assert np.all(r.margin == 0.0)


def test_gamma_monotone_and_extremes(oracle_lib):
    """A smaller gamma accepts a superset; gamma = 0 accepts every in-range
    draft (accept length K, bonus-row token); a huge gamma rejects the first
    draft (accept length 0, token of row 0)."""
    a, b, t, d = _rows(6, 3, 200, 3)
    prev = None
    for g in (4.0, 1.0, 0.5, 0.1):
        r = _asym(a, b, t, d, gamma=g)
        if prev is not None:
            assert np.all(r.accept >= prev.accept)
            assert np.all(r.accept_len >= prev.accept_len)
        prev = r
    r0 = _asym(a, b, t, d, gamma=0.0)
    assert np.all(r0.accept == 1) and np.all(r0.accept_len == 3)
    np.testing.assert_array_equal(r0.token, r0.fused[:, 3])
    rh = _asym(a, b, t, d, gamma=1e30)
    assert np.all(rh.accept == 0) and np.all(rh.accept_len == 0)
    np.testing.assert_array_equal(rh.token, rh.fused[:, 0])


def test_scan_first_rejection(oracle_lib):
    """Emission at the first rejection (AsymSpec notes 4.2) on a constructed
    pattern: rows 0 and 2 accept, row 1 rejects -> length 1, token of row 1."""
    V = 4
    t = np.zeros((1, 4, V), np.float32)
    b = np.zeros((1, 4, V), np.float32)
    a = np.zeros((1, 4, V), np.float32)
    t[0, 0, 0] = 3.0           # draft 0 strongly favoured by the verifier
    t[0, 1, 0] = -3.0          # draft 0 disfavoured
    t[0, 2, 0] = 3.0
    t[0, 1, 2] = 1.0           # row 1's fused token is 2
    d = np.zeros((1, 3), np.int32)
    r = _asym(a, b, t, d, beta=1.0, gamma=0.5)
    np.testing.assert_array_equal(r.accept[0], [1, 0, 1])
    assert r.accept_len[0] == 1 and r.token[0] == 2


def test_beta_does_not_change_gate(oracle_lib):
    """D, gamma_eff, accept and the accept length do not depend on beta
    (beta only enters the fused token, AsymSpec notes 4.1-4.2)."""
    x = W.gen_asym(4, 2, 2048, "bf16", seed=5)
    rs = [_asym(x.a, x.b, x.t, x.draft, beta=bt, gamma=0.5, dtype="bf16") for bt in (0.0, 1.0, 2.0)]
    for r in rs[1:]:
        np.testing.assert_array_equal(r.D, rs[0].D)
        np.testing.assert_array_equal(r.gamma_eff, rs[0].gamma_eff)
        np.testing.assert_array_equal(r.accept, rs[0].accept)
        np.testing.assert_array_equal(r.accept_len, rs[0].accept_len)


def test_standard_verification_point(oracle_lib):
    """beta=0, gamma=1 (AsymSpec notes 4.2): the emitted-token rule becomes
    argmax t, the CDA test accepts a superset of the fixed test
    p_t(d) > p_b(d), and the two agree wherever D = 0."""
    pt = GOLDEN["standard_verification_point"]["value"]
    x = W.gen_asym(16, 2, 1024, "bf16", seed=12, identical_frac=0.3)
    r = _asym(x.a, x.b, x.t, x.draft, beta=pt["beta"], gamma=pt["gamma"], dtype="bf16")
    np.testing.assert_array_equal(r.fused, np.argmax(x.t, axis=2))
    for bi in range(x.B):
        for i in range(x.K):
            dd = x.draft[bi, i]
            std = softmax(x.t[bi, i].astype(np.float64))[dd] > softmax(x.b[bi, i].astype(np.float64))[dd]
            assert (not std) or r.accept[bi, i]
            if x.identical[bi, i]:
                assert bool(r.accept[bi, i]) == bool(std)


def test_bad_draft_is_rejected(oracle_lib):
    a, b, t, d = _rows(2, 2, 16, 1)
    d[0, 0] = 16
    d[1, 1] = -1
    r = _asym(a, b, t, d, gamma=0.0)
    assert r.accept[0, 0] == 0 and r.accept[1, 1] == 0
    assert r.accept_len[0] == 0 and r.accept_len[1] == 1


# ------------------------------------------------ AsymSpec ablation variants
# The mechanism ablation of the AsymSpec notes (experiments; counterfactual
# reasoning) swaps the fusion source for the raw full-context logits a or for
# the two-model difference t - b, and replaces the CDA threshold by a fixed
# gamma (the gate section 4.2 argues against).

def test_delta_raw_a_follows_a_alone(oracle_lib):
    """delta = a: with a flat verifier row the fused token is argmax a (beta
    > 0) or argmin a (beta < 0), lowest index first; b never matters."""
    a, b, t, d = _rows(4, 2, 257, 31)
    flat = np.zeros_like(t)
    r = oracle.asym(a, b, flat, d, 1.5, 0.5, "f32", delta="a")
    np.testing.assert_array_equal(r.fused, np.argmax(a, axis=2))
    r = oracle.asym(a, b, flat, d, -0.75, 0.5, "f32", delta="a")
    np.testing.assert_array_equal(r.fused, np.argmin(a, axis=2))
    r1 = oracle.asym(a, b, t, d, 1.0, 0.5, "f32", delta="a")
    b2 = np.random.default_rng(5).normal(0, 3, size=b.shape).astype(np.float32)
    r2 = oracle.asym(a, b2, t, d, 1.0, 0.5, "f32", delta="a")
    np.testing.assert_array_equal(r1.fused, r2.fused)
    np.testing.assert_array_equal(r1.top, r2.top)
    # the default source does depend on b
    r3 = oracle.asym(a, b, t, d, 1.0, 0.5, "f32")
    r4 = oracle.asym(a, b2, t, d, 1.0, 0.5, "f32")
    assert np.any(r3.fused != r4.fused)


def test_delta_two_model_difference(oracle_lib):
    """delta = t - b: at beta = -1 the score t - (t - b) is b, so the fused
    token is argmax b; with b equal to t it is argmax t; a never matters."""
    a, b, t, d = _rows(4, 2, 300, 32, dyadic=True)
    r = oracle.asym(a, b, t, d, -1.0, 0.5, "f32", delta="t-b")
    np.testing.assert_array_equal(r.fused, np.argmax(b, axis=2))
    r = oracle.asym(a, t.copy(), t, d, 2.0, 0.5, "f32", delta="t-b")
    np.testing.assert_array_equal(r.fused, np.argmax(t, axis=2))
    r1 = oracle.asym(a, b, t, d, 1.0, 0.5, "f32", delta="t-b")
    a2 = np.random.default_rng(6).normal(0, 3, size=a.shape).astype(np.float32)
    r2 = oracle.asym(a2, b, t, d, 1.0, 0.5, "f32", delta="t-b")
    np.testing.assert_array_equal(r1.fused, r2.fused)
    np.testing.assert_array_equal(r1.gap, r2.gap)


def test_delta_sources_coincide_where_they_must(oracle_lib):
    """With a := t the context gain a - b is the two-model difference t - b;
    with b := 0 it is the raw a.  Scores agree bit for bit there."""
    a, b, t, d = _rows(3, 2, 500, 33)
    r1 = oracle.asym(t.copy(), b, t, d, 1.3, 0.5, "f32", delta="a-b")
    r2 = oracle.asym(a, b, t, d, 1.3, 0.5, "f32", delta="t-b")
    np.testing.assert_array_equal(r1.fused, r2.fused)
    np.testing.assert_array_equal(r1.top, r2.top)
    np.testing.assert_array_equal(r1.gap, r2.gap)
    zero = np.zeros_like(b)
    r3 = oracle.asym(a, zero, t, d, 1.3, 0.5, "f32", delta="a-b")
    r4 = oracle.asym(a, b, t, d, 1.3, 0.5, "f32", delta="a")
    np.testing.assert_array_equal(r3.fused, r4.fused)
    np.testing.assert_array_equal(r3.top, r4.top)


def test_fixed_gate_matches_scipy(oracle_lib):
    """The fixed gate accepts iff softmax(t)[d] > gamma * softmax(b)[d]; its
    margin is the log-space difference against log gamma; the threshold it
    reports is gamma itself; D is still the CDA divergence; a does not enter."""
    a, b, t, d = _rows(6, 3, 700, 34)
    gamma = 0.6
    r = oracle.asym(a, b, t, d, 1.0, gamma, "f32", gate="fixed")
    rc = oracle.asym(a, b, t, d, 1.0, gamma, "f32")
    g32 = float(np.float32(gamma))
    assert np.all(r.gamma_eff == g32)
    np.testing.assert_array_equal(r.D, rc.D)
    for bi in range(6):
        for i in range(3):
            dd = d[bi, i]
            lt = log_softmax(t[bi, i].astype(np.float64))[dd]
            lb = log_softmax(b[bi, i].astype(np.float64))[dd]
            assert abs(r.margin[bi, i] - (lt - lb - math.log(g32))) < 1e-12
            pt = softmax(t[bi, i].astype(np.float64))[dd]
            pb = softmax(b[bi, i].astype(np.float64))[dd]
            assert bool(r.accept[bi, i]) == bool(pt > g32 * pb)
    a2 = np.random.default_rng(7).normal(0, 3, size=a.shape).astype(np.float32)
    r2 = oracle.asym(a2, b, t, d, 1.0, gamma, "f32", gate="fixed")
    np.testing.assert_array_equal(r2.accept, r.accept)
    np.testing.assert_array_equal(r2.margin, r.margin)
    assert np.any(r2.D != r.D)


def test_fixed_gate_against_cda(oracle_lib):
    """D >= 0 makes the CDA threshold gamma*exp(-D) no larger than gamma: every
    draft the fixed gate accepts, CDA accepts too; they agree where D = 0; the
    gate never moves the fused token."""
    x = W.gen_asym(24, 3, 1024, "bf16", seed=35, identical_frac=0.3, displaced_frac=0.5)
    x.draft = np.random.default_rng(8).integers(0, 1024, size=x.draft.shape).astype(np.int32)
    for delta in ("a-b", "a", "t-b"):
        rf = oracle.asym(x.a, x.b, x.t, x.draft, 1.0, 0.5, "bf16", delta=delta, gate="fixed")
        rc = oracle.asym(x.a, x.b, x.t, x.draft, 1.0, 0.5, "bf16", delta=delta)
        assert np.all(rc.accept >= rf.accept)
        ident = x.identical[:, :x.K]
        np.testing.assert_array_equal(rf.accept[ident], rc.accept[ident])
        np.testing.assert_array_equal(rf.fused, rc.fused)
    assert np.any(rc.accept > rf.accept)  # CDA does relax somewhere on these rows


# ------------------------------------------------ AsymSpec from hidden states
# The step before the pass on the AsymSpec pages: the logits are the LM
# heads' products of the hidden states.

def test_lmhead_identity_heads_reduce_to_the_pass(oracle_lib):
    """With H = V and scaled identity heads the logits are c*h exactly, and
    the LM-head oracle is the AsymSpec oracle on those rows, bit for bit."""
    x = W.gen_asym(3, 2, 96, "bf16", seed=70, identical_frac=0.2, tie_frac=0.3)
    for c in (1.0, 2.0):
        Wh = (c * np.eye(96)).astype(np.float32)
        r = oracle.asym_lmhead(x.a, x.b, Wh, x.t, Wh, x.draft, 1.0, 0.5).res
        ref = oracle.asym(c * x.a, c * x.b, c * x.t, x.draft, 1.0, 0.5, "f32")
        for f in ("lse", "D", "gamma_eff", "fused", "gap", "top", "accept", "margin", "accept_len", "token"):
            np.testing.assert_array_equal(getattr(r, f), getattr(ref, f), err_msg=f)
        rf = oracle.asym_lmhead(x.a, x.b, Wh, x.t, Wh, x.draft, 1.0, 0.5, gate="fixed").res
        np.testing.assert_array_equal(rf.accept, oracle.asym(c * x.a, c * x.b, c * x.t, x.draft, 1.0, 0.5, "f32",
                                                             gate="fixed").accept)


def test_lmhead_error_bound_covers_fp32_sums(oracle_lib):
    """The reported bound on an fp32 product-sum of the heads covers the
    actual error of fp32 matrix products (two summation orders) of the same
    inputs."""
    x = W.gen_lmhead(2, 2, 700, 512, seed=71)
    r = oracle.asym_lmhead(x.h_a, x.h_b, x.W_d, x.h_t, x.W_t, x.draft, 1.0, 0.5)
    ha = x.h_a.reshape(-1, x.Hd)
    exact = ha.astype(np.float64) @ x.W_d.astype(np.float64).T
    f32 = (ha @ x.W_d.T).astype(np.float64)
    seq = np.zeros((ha.shape[0], x.V), np.float32)
    for k in range(x.Hd):          # one product at a time: the longest chain of roundings
        seq = (seq + np.outer(ha[:, k], x.W_d[:, k])).astype(np.float32)
    err = r.err_a.reshape(-1)
    assert np.all(np.abs(f32 - exact).max(axis=1) <= err)
    assert np.all(np.abs(seq.astype(np.float64) - exact).max(axis=1) <= err)
    assert np.all(err < 1e-2)


def test_lmhead_dyadic_products_are_exact(oracle_lib):
    """With signed power-of-two entries every fp32 summation order of the
    head products gives the fp64 logits exactly (checked on three orders),
    and the oracle reports a zero bound for them."""
    x = W.gen_lmhead_dyadic(2, 2, 300, 512, seed=72)
    r = oracle.asym_lmhead(x.h_a, x.h_b, x.W_d, x.h_t, x.W_t, x.draft, 1.0, 0.5)
    for h, Wm in ((x.h_a, x.W_d), (x.h_b, x.W_d), (x.h_t, x.W_t)):
        hh = h.reshape(-1, h.shape[-1])
        exact = hh.astype(np.float64) @ Wm.astype(np.float64).T
        np.testing.assert_array_equal((hh @ Wm.T).astype(np.float64), exact)
        for order in (range(hh.shape[1]), range(hh.shape[1] - 1, -1, -1)):
            seq = np.zeros(exact.shape, np.float32)
            for k in order:
                seq = (seq + np.outer(hh[:, k], Wm[:, k])).astype(np.float32)
            np.testing.assert_array_equal(seq.astype(np.float64), exact)
    for e in (r.err_a, r.err_b, r.err_t, r.err_bd, r.err_td):
        assert np.all(e == 0.0)
    # the planted structure survives: spikes make the drafts the drafter's top tokens
    a = x.h_a.reshape(-1, x.Hd).astype(np.float64) @ x.W_d.astype(np.float64).T
    top = a.reshape(x.B, x.K + 1, x.V)[:, :x.K].argmax(axis=2)
    assert np.mean(top == x.draft) > 0.8


def test_lmhead_bound_nonzero_when_a_sum_can_round(oracle_lib):
    """One fine entry among coarse ones: 32 ones and 2^-20 need 26 significant
    bits, an fp32 order that adds the fine term last rounds it away, and the
    oracle's bound must be nonzero and cover that error."""
    n = 32
    h = np.ones((1, 2, n), np.float32)
    h[0, 0, 0] = 2.0 ** -20
    Wm = np.ones((2, n), np.float32)
    r = oracle.asym_lmhead(h, h, Wm, h, Wm, np.zeros((1, 1), np.int32), 1.0, 0.5)
    exact = 31.0 + 2.0 ** -20
    rounded = float(np.float32(np.float32(31.0) + np.float32(2.0 ** -20)))
    assert rounded != exact
    assert r.err_a[0, 0] >= abs(rounded - exact) > 0.0
    # a row of ones only (no fine term) is exact again
    assert r.err_a[0, 1] > 0.0          # the bound is per call: q is the finest bit of all of h
    h2 = np.ones((1, 2, n), np.float32)
    r2 = oracle.asym_lmhead(h2, h2, Wm, h2, Wm, np.zeros((1, 1), np.int32), 1.0, 0.5)
    assert np.all(r2.err_a == 0.0)
    # products that underflow fp32 (2^-80 * 2^-80) are not exact: the bound stays
    tiny = np.full((1, 2, n), 2.0 ** -80, np.float32)
    Wt = np.full((2, n), 2.0 ** -80, np.float32)
    r3 = oracle.asym_lmhead(tiny, tiny, Wt, tiny, Wt, np.zeros((1, 1), np.int32), 1.0, 0.5)
    assert np.all(r3.err_a > 0.0)
    assert float(np.float32(2.0 ** -80) * np.float32(2.0 ** -80)) == 0.0


# ------------------------------------------------ AsymSpec across model families
# AsymSpec notes, the analysis of cross-family pairs: the drafter's gain
# reaches the verifier through a vocabulary alignment of string-identical
# tokens, generation restricted to that shared subset.

def test_xfam_identity_alignment_is_the_same_family_pass(oracle_lib):
    """With one vocabulary and the identity alignment the cross-family pass
    is the AsymSpec pass, bit for bit."""
    x = W.gen_asym(5, 3, 777, "bf16", seed=60, identical_frac=0.2, tie_frac=0.2)
    vmap = np.arange(777, dtype=np.int32)
    r1 = oracle.asym_xfam(x.a, x.b, x.t, vmap, x.draft, 1.25, 0.5, "bf16")
    r2 = oracle.asym(x.a, x.b, x.t, x.draft, 1.25, 0.5, "bf16")
    for f in ("lse", "D", "gamma_eff", "fused", "gap", "top", "accept", "margin", "accept_len", "token"):
        np.testing.assert_array_equal(getattr(r1, f), getattr(r2, f), err_msg=f)


def test_xfam_relabelled_verifier_vocabulary(oracle_lib):
    """Relabelling the verifier vocabulary (t'[v] = t[perm[v]], alignment
    v -> perm[v], drafts mapped back) relabels the fused token and leaves
    every other output unchanged."""
    a, b, t, d = _rows(3, 2, 400, 61)
    perm = np.random.default_rng(62).permutation(400).astype(np.int32)
    inv = np.argsort(perm).astype(np.int32)
    r1 = oracle.asym(a, b, t, d, 0.8, 0.6, "f32")
    r2 = oracle.asym_xfam(a, b, np.ascontiguousarray(t[:, :, perm]), perm, inv[d], 0.8, 0.6, "f32")
    np.testing.assert_array_equal(perm[r2.fused], r1.fused)
    for f in ("D", "gamma_eff", "accept", "accept_len"):
        np.testing.assert_array_equal(getattr(r1, f), getattr(r2, f), err_msg=f)
    np.testing.assert_allclose(r2.margin, r1.margin, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r2.lse, r1.lse, rtol=0, atol=1e-12)


def test_xfam_unpaired_tokens_are_never_emitted_or_accepted(oracle_lib):
    """Generation is restricted to the paired tokens: a verifier token with
    no drafter pair is never the fused token, however large its logit, and a
    draft on it is rejected; with no pair at all there is no fused token."""
    x = W.gen_xfam(3, 2, 500, 450, 300, "f32", seed=63)
    free = np.flatnonzero(x.vmap < 0)
    t = x.t.copy()
    t[:, :, free[0]] = 1e4
    r = oracle.asym_xfam(x.a, x.b, t, x.vmap, x.draft, 1.0, 0.5, "f32")
    assert np.all(x.vmap[r.fused] >= 0)
    # the maximum over paired tokens, by brute force on the stored values
    for bi in range(3):
        for i in range(3):
            s64 = np.full(450, -np.inf)
            ok = x.vmap >= 0
            e = x.vmap[ok]
            s64[ok] = t[bi, i, ok].astype(np.float64) + (x.a[bi, i, e].astype(np.float64) - x.b[bi, i, e])
            assert r.fused[bi, i] == int(np.argmax(s64))
    d = x.draft.copy()
    d[0, 0] = free[1]
    r2 = oracle.asym_xfam(x.a, x.b, t, x.vmap, d, 1.0, 0.0, "f32")
    assert r2.accept[0, 0] == 0 and np.isnan(r2.margin[0, 0]) and r2.accept_len[0] == 0
    r3 = oracle.asym_xfam(x.a, x.b, t, np.full(450, -1, np.int32), x.draft, 1.0, 0.5, "f32")
    assert np.all(r3.fused == -1) and np.all(r3.token == -1) and np.all(r3.accept == 0)


def test_xfam_acceptance_against_scipy(oracle_lib):
    """The test compares the verifier's probability of the draft with the
    drafter's compressed-view probability of its pair."""
    x = W.gen_xfam(4, 3, 600, 550, 400, "f32", seed=64)
    r = oracle.asym_xfam(x.a, x.b, x.t, x.vmap, x.draft, 1.0, 0.5, "f32")
    for j, v in enumerate((x.a, x.b, x.t)):   # each normaliser over its own vocabulary
        np.testing.assert_allclose(r.lse[..., j], logsumexp(v.astype(np.float64), axis=2), rtol=0, atol=1e-12)
    for bi in range(4):
        for i in range(3):
            dv = x.draft[bi, i]
            e = x.vmap[dv]
            lt = log_softmax(x.t[bi, i].astype(np.float64))[dv]
            lb = log_softmax(x.b[bi, i].astype(np.float64))[e]
            p = softmax(x.a[bi, i].astype(np.float64))
            q = softmax(x.b[bi, i].astype(np.float64))
            Dj = jensenshannon(p, q) ** 2
            want = lt - lb - math.log(float(np.float32(0.5))) + Dj
            assert abs(r.margin[bi, i] - want) < 1e-9
            assert bool(r.accept[bi, i]) == (want > 0)


# ------------------------------------------------ E2-SCI adaptive acceptance
# E2-SCI notes, key design 3: per-position JSD of drafter and target against
# the window's threshold, the EWMA credit state and the clamped threshold.

def _e2sci_rows(B, Wn, V, seed, scale=2.0):
    rng = np.random.default_rng(seed)
    y = rng.normal(0, scale, size=(B, Wn, V)).astype(np.float32)
    z = (y + rng.normal(0, 0.7, size=y.shape)).astype(np.float32)
    return y, z


@pytest.mark.parametrize("V", [2, 7, 1000])
def test_e2sci_jsd_matches_scipy(oracle_lib, V):
    y, z = _e2sci_rows(3, 4, V, 40 + V)
    r = oracle.e2sci(y, z, np.full(3, 0.1), np.ones(3), np.full(3, 0.5))
    for bi in range(3):
        for i in range(4):
            p = softmax(y[bi, i].astype(np.float64))
            q = softmax(z[bi, i].astype(np.float64))
            assert abs(r.D[bi, i] - jensenshannon(p, q) ** 2) <= 1e-12 + 1e-10 * r.D[bi, i]


def test_e2sci_threshold_is_inclusive(oracle_lib):
    """A divergence above the threshold rejects, one equal to it does not:
    identical rows (D = 0) pass at T = 0; a row passes at the float32 just
    above its D and fails at the one just below."""
    y, z = _e2sci_rows(2, 3, 300, 41)
    z[0] = y[0]
    r = oracle.e2sci(y, z, np.zeros(2, np.float32), np.ones(2), np.full(2, 0.5))
    assert np.all(r.D[0] == 0.0) and np.all(r.accept[0] == 1) and r.accept_len[0] == 3
    assert np.all(r.D[1] > 0.0) and np.all(r.accept[1] == 0) and r.accept_len[1] == 0
    d = r.D[1, 0]
    up = np.nextafter(np.float32(d), np.float32(1.0))
    dn = np.nextafter(np.float32(d), np.float32(0.0))
    assert r.accept[1, 0] == 0
    ru = oracle.e2sci(y, z, np.array([0.0, up], np.float32), np.ones(2), np.full(2, 0.5))
    rd = oracle.e2sci(y, z, np.array([0.0, dn], np.float32), np.ones(2), np.full(2, 0.5))
    assert ru.accept[1, 0] == 1 and rd.accept[1, 0] == 0


def test_e2sci_scan_stops_at_first_rejection(oracle_lib):
    y, z = _e2sci_rows(1, 6, 500, 42)
    z[0, [0, 1, 3]] = y[0, [0, 1, 3]]      # D = 0 at positions 0, 1, 3
    r = oracle.e2sci(y, z, np.zeros(1, np.float32), np.ones(1), np.full(1, 0.5))
    np.testing.assert_array_equal(r.accept[0], [1, 1, 0, 1, 0, 0])
    assert r.accept_len[0] == 2


def test_e2sci_ewma_closed_form(oracle_lib):
    """With every window fully accepted (T above ln 2) the credit state follows
    r_n = 1 - (1 - r_0)(1 - beta)^n; fully rejected (T below 0), r_0 (1 - beta)^n;
    beta = 0.3 as printed on the page."""
    beta = GOLDEN["e2sci_ewma"]["value"]
    prm = oracle.E2sciParams(ewma=beta)
    y, z = _e2sci_rows(2, 4, 64, 43)
    r0 = np.array([0.2, 0.9], np.float32)
    for T, target in ((1.0, 1.0), (-1.0, 0.0)):
        r = r0.copy()
        for n in range(1, 6):
            out = oracle.e2sci(y, z, np.full(2, T, np.float32), np.ones(2), r, prm)
            r = out.r_hat.astype(np.float32)
            want = target + (r0.astype(np.float64) - target) * (1 - beta) ** n
            np.testing.assert_allclose(out.r_hat, want, rtol=0, atol=1e-6)
    # a half-accepted window moves r halfway by beta
    z2 = z.copy()
    z2[0, :2] = y[0, :2]
    out = oracle.e2sci(y, z2, np.zeros(2, np.float32), np.ones(2), np.array([0.0, 0.0], np.float32), prm)
    assert out.accept_len[0] == 2 and abs(out.r_hat[0] - float(np.float32(beta)) * 0.5) < 1e-15


def test_e2sci_threshold_update(oracle_lib):
    """Delta T = alpha * omega * (r - tau): positive above the neutral credit,
    negative below, linear in omega; the result is clamped to [T_min, T_max]."""
    prm = oracle.E2sciParams(alpha=0.5, tau_credit=0.5, T_base=0.1, T_min=0.02, T_max=0.25, ewma=1.0)
    y, z = _e2sci_rows(4, 4, 64, 44)
    z[:2] = y[:2]                          # requests 0, 1 accept everything: r = 1
    T_in = np.zeros(4, np.float32)
    omega = np.array([0.2, 0.4, 0.2, 0.4], np.float32)
    out = oracle.e2sci(y, z, T_in, omega, np.zeros(4, np.float32), prm)
    np.testing.assert_array_equal(out.accept_len, [4, 4, 0, 0])
    f = lambda v: float(np.float32(v))
    for bi in range(4):
        r = float(out.r_hat[bi])
        want = f(0.1) + f(0.5) * float(omega[bi]) * (r - f(0.5))
        assert abs(out.T_next[bi] - min(max(want, f(0.02)), f(0.25))) < 1e-12
    assert out.T_next[0] > f(0.1) and out.T_next[2] < f(0.1)
    assert abs((out.T_next[1] - f(0.1)) - 2 * (out.T_next[0] - f(0.1))) < 1e-9
    big = oracle.e2sci(y, z, T_in, np.full(4, 100.0, np.float32), np.zeros(4, np.float32), prm)
    np.testing.assert_array_equal(big.T_next, [f(0.25), f(0.25), f(0.02), f(0.02)])


# The stabilisers of the same passage (hysteresis, a minimum refresh
# interval, a safety fall-back when the acceptance drops below delta): the
# page names them without a rule; the oracle's reading is pinned on
# constructed sequences whose outcome follows from that reading by hand.

def test_e2sci_stabilisers_off_by_default(oracle_lib):
    """Default constants leave the page's update untouched: the next threshold
    is the clamped proposal on every request, whatever the age."""
    y, z = _e2sci_rows(6, 4, 200, 45)
    z[:2] = y[:2]
    rng = np.random.default_rng(45)
    T_in = rng.uniform(0.0, 0.3, 6).astype(np.float32)
    out = oracle.e2sci(y, z, T_in, np.ones(6, np.float32), np.full(6, 0.5, np.float32),
                       age=np.array([0, 1, 5, 0, 7, 2]))
    np.testing.assert_array_equal(out.T_next, out.T_prop)
    assert np.all((out.age == 0) | (out.T_prop == T_in.astype(np.float64)))


def test_e2sci_hysteresis_dead_band():
    """A proposal within the dead band of the current threshold (either side)
    keeps it; one beyond it is adopted, and the age restarts."""
    f = lambda v: float(np.float32(v))
    prm = oracle.E2sciParams(hysteresis=0.005)
    T0 = f(0.1)
    for dT, moves in ((0.0049, False), (-0.0049, False), (0.0051, True), (-0.0051, True)):
        T, age, m = oracle.e2sci_stabilise(T0, T0 + dT, 0.5, 3, prm)
        assert (T != T0) == moves and (age == 0) == moves, dT
        assert T == (T0 + dT if moves else T0)
        assert abs(m - (abs(dT) - f(0.005))) < 1e-12
    # a proposal oscillating by +-0.003 around the threshold never moves it
    # with a 0.005 band; with a 0.002 band it follows every proposal
    props = [T0 + (0.003 if k % 2 else -0.003) for k in range(8)]
    for band, follows in ((0.005, False), (0.002, True)):
        T, age = T0, 0
        seen = []
        for pr in props:
            T, age, _ = oracle.e2sci_stabilise(T, pr, 0.5, age, oracle.E2sciParams(hysteresis=band))
            seen.append(T)
        assert seen == (props if follows else [T0] * 8)


def test_e2sci_minimum_refresh_interval():
    """With a minimum interval of 3 windows a threshold set at age 0 holds for
    two more windows and the proposal is adopted on the third; a fresh
    proposal on every window therefore lands on windows 3, 6, 9."""
    prm = oracle.E2sciParams(min_refresh=3)
    T, age = 0.1, 0
    changes = []
    for k in range(1, 10):
        T_new, age, _ = oracle.e2sci_stabilise(T, 0.1 + 0.01 * k, 0.5, age, prm)
        if T_new != T:
            changes.append(k)
        T = T_new
    assert changes == [3, 6, 9]
    # min_refresh 0 or 1: every window may refresh
    for m in (0, 1):
        T, age, _ = oracle.e2sci_stabilise(0.1, 0.2, 0.5, 0, oracle.E2sciParams(min_refresh=m))
        assert T == 0.2 and age == 0


def test_e2sci_safety_fallback():
    """An accepted fraction below delta sets the conservative threshold at
    once, inside the refresh interval and inside the dead band; one equal to
    delta does not trigger it."""
    f = lambda v: float(np.float32(v))
    prm = oracle.E2sciParams(hysteresis=0.5, min_refresh=5, delta=0.25, T_safe=0.02)
    T, age, m = oracle.e2sci_stabilise(0.1, 0.1, 0.125, 0, prm)
    assert T == f(0.02) and age == 0 and np.isnan(m)
    T, age, _ = oracle.e2sci_stabilise(0.1, 0.3, 0.25, 0, prm)     # p_acc == delta: interval holds
    assert T == 0.1 and age == 1


def test_e2sci_stabilised_window(oracle_lib):
    """End to end on rows: requests whose drafter equals the target accept
    the whole window (p_acc = 1) and get the proposal (outside the band);
    requests that reject at once (p_acc = 0 < delta) fall back to T_safe;
    a request still inside its refresh interval keeps its threshold."""
    f = lambda v: float(np.float32(v))
    prm = oracle.E2sciParams(alpha=0.5, tau_credit=0.5, T_base=0.1, T_min=0.02, T_max=0.25, ewma=1.0,
                             hysteresis=0.01, min_refresh=2, delta=0.5, T_safe=0.03)
    y, z = _e2sci_rows(4, 4, 64, 46)
    z[[0, 3]] = y[[0, 3]]
    T_in = np.zeros(4, np.float32)
    out = oracle.e2sci(y, z, T_in, np.ones(4, np.float32), np.zeros(4, np.float32), prm,
                       age=np.array([1, 1, 0, 0]))
    np.testing.assert_array_equal(out.accept_len, [4, 0, 0, 4])
    assert out.T_prop[0] == f(0.25)                          # 0.1 + 0.5 * (1 - 0.5), clamped to T_max
    assert out.T_next[0] == f(0.25) and out.age[0] == 0
    assert out.T_next[1] == f(0.03) and out.T_next[2] == f(0.03) and out.age[1] == out.age[2] == 0
    assert out.T_next[3] == 0.0 and out.age[3] == 1          # age 0 + 1 < 2: held


def test_page_defaults_in_workloads():
    """The named workloads use the pages' hyperparameters (AsymSpec notes 4.4;
    RAPID notes, hyperparameters)."""
    x = W.tiny_asym()
    assert x.K == GOLDEN["asym_K"]["value"]
    assert x.beta == GOLDEN["asym_beta"]["value"] and x.gamma == GOLDEN["asym_gamma"]["value"]
    assert W.C3_ETAS == tuple(float(e) for e in GOLDEN["rapid_eta_self"]["value"])
    r = W.gen_rapid(2, GOLDEN["rapid_drafts"]["value"], 64, seed=1)
    assert r.G == 10


# ---------------------------------------------------------------- RAPID
def _kd_loss(z, y, T):
    """T^2 * KL(q || softmax(z/T)) with q = softmax(y/T)."""
    q = softmax(y / T)
    return T * T * float(np.sum(q * (np.log(q) - log_softmax(z / T))))


@pytest.mark.parametrize("T", [1.0, 0.7, 2.0])
def test_zhat_is_one_kd_gradient_step(oracle_lib, T):
    """RAPID notes design 2: zhat = z - eta * dL/dz with L = T^2 KL(q||p),
    checked by central finite differences of L built from scipy routines."""
    rng = np.random.default_rng(int(T * 10))
    V = 12
    z = rng.normal(0, 2, V)
    y = rng.normal(0, 2, V)
    eta = 5.0
    h = 1e-5
    grad = np.zeros(V)
    for v in range(V):
        e = np.zeros(V)
        e[v] = h
        grad[v] = (_kd_loss(z + e, y, T) - _kd_loss(z - e, y, T)) / (2 * h)
    zhat = oracle.rapid_zhat(z, y, eta, T)
    np.testing.assert_allclose(zhat, z - eta * grad, rtol=0, atol=1e-7)


def test_eta_zero_is_plain_target(oracle_lib):
    """eta = 0: zhat = z, so phat = p and tail protection changes nothing."""
    rng = np.random.default_rng(4)
    z = rng.normal(0, 2, 50)
    y = rng.normal(0, 2, 50)
    np.testing.assert_array_equal(oracle.rapid_zhat(z, y, 0.0, 1.3), z)
    np.testing.assert_allclose(oracle.rapid_phat(z, y, 0.0, 1.3), softmax(z / 1.3), rtol=1e-13)


def test_tail_protection_constructed(oracle_lib):
    """RAPID notes design 3: tokens whose augmented probability is below 10%
    of the peak keep the original target probability; the others take the
    augmented one.  Row built so that tokens 2..5 are far below the peak."""
    z = np.array([0.0, -0.5, -6.0, -7.0, -8.0, -9.0])
    y = np.array([-0.5, 0.0, -9.0, -6.0, -8.0, -7.0])
    eta, T = 3.0, 1.0
    zhat = oracle.rapid_zhat(z, y, eta, T)
    raw = softmax(zhat / T)
    assert np.all(raw[2:] < 0.1 * raw.max()) and np.all(raw[:2] >= 0.1 * raw.max())
    ph = oracle.rapid_phat(z, y, eta, T)
    np.testing.assert_allclose(ph[2:], softmax(z / T)[2:], rtol=1e-13)
    np.testing.assert_allclose(ph[:2], raw[:2], rtol=1e-13)
    # the protected target is not renormalised
    assert abs(ph.sum() - 1.0) > 1e-6


def test_equal_target_and_drafter_is_noop(oracle_lib):
    """q = p: no knowledge to transfer, zhat = z and phat = p."""
    rng = np.random.default_rng(8)
    z = rng.normal(0, 2, 40)
    np.testing.assert_allclose(oracle.rapid_zhat(z, z.copy(), 20.0, 1.0), z, atol=1e-13)
    np.testing.assert_allclose(oracle.rapid_phat(z, z.copy(), 20.0, 1.0), softmax(z), rtol=1e-12)


def _rapid_one(z_rows, y_rows, draft, ua, us, eta, T, want_dist=False):
    z = np.asarray(z_rows, np.float32)[None]
    y = np.asarray(y_rows, np.float32)[None]
    return oracle.rapid(z, y, np.asarray(draft, np.int32)[None], np.asarray(ua, np.float32)[None],
                        np.asarray(us, np.float32)[None], eta, T, want_dist=want_dist)


def test_inverse_cdf_draw_constructed(oracle_lib):
    """Residual draw on a hand-built row (eta = 0): p = (.1,.2,.3,.4),
    q = (.4,.3,.2,.1), residual max(p - q, 0) = (0, 0, .1, .3), S = .4.
    Vocabulary-order inverse CDF: u*S below .1 -> token 2, above -> token 3."""
    p = np.log(np.array([0.1, 0.2, 0.3, 0.4]))
    q = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    rows_z = [p, p]
    rows_y = [q, q]
    for u, tok in [(0.0, 2), (0.2, 2), (0.24, 2), (0.26, 3), (0.9, 3)]:
        r = _rapid_one(rows_z, rows_y, [9], [0.0], [u, 0.0], 0.0, 1.0, want_dist=True)
        # draft id 9 is outside the vocabulary: rejected, draw from row 0's residual
        assert r.accept_len[0] == 0
        assert r.token[0] == tok
        assert r.resid_S[0] == pytest.approx(0.4, rel=1e-6)
        np.testing.assert_allclose(r.emit_dist[0], [0, 0, 0.25, 0.75], atol=1e-6)


def test_bonus_row_draws_from_target(oracle_lib):
    """All G drafts accepted: the extra token comes from p of the last row,
    checked with numpy's searchsorted over scipy's softmax."""
    rng = np.random.default_rng(21)
    G, V = 3, 30
    z = rng.normal(0, 1, (G + 1, V)).astype(np.float32)
    y = rng.normal(0, 1, (G + 1, V)).astype(np.float32)
    for u in (0.05, 0.5, 0.93):
        r = _rapid_one(z, y, [1, 2, 3], [0.0] * G, [0.1] * G + [u], 7.0, 1.0)
        assert r.accept_len[0] == G and r.resid_S[0] == -1.0
        p = softmax(z[G].astype(np.float64))
        assert r.token[0] == int(np.searchsorted(np.cumsum(p), u * p.sum(), side="right"))


def test_zero_residual_falls_back_to_target(oracle_lib):
    """p = q and eta = 0: the residual is identically 0, so the draw uses p."""
    rng = np.random.default_rng(2)
    z = rng.normal(0, 1, (2, 16)).astype(np.float32)
    r = _rapid_one(z, z, [99], [0.0], [0.6, 0.1], 0.0, 1.0)
    assert r.accept_len[0] == 0 and r.resid_S[0] == -1.0
    p = softmax(z[0].astype(np.float64))
    assert r.token[0] == int(np.searchsorted(np.cumsum(p), 0.6 * p.sum(), side="right"))


def test_temperature_placement(oracle_lib):
    """p = softmax(z/T), q = softmax(y/T) and phat = softmax(zhat/T): running
    with (z, y, T=2) equals running with (z/2, y/2, T=1)."""
    rng = np.random.default_rng(13)
    G, V = 4, 64
    z = (np.round(rng.normal(0, 2, (3, G + 1, V)) * 256) / 256).astype(np.float32)
    y = (np.round(rng.normal(0, 2, (3, G + 1, V)) * 256) / 256).astype(np.float32)
    d = rng.integers(0, V, (3, G)).astype(np.int32)
    ua = W.uniforms_2p24(rng, (3, G))
    us = W.uniforms_2p24(rng, (3, G + 1))
    r2 = oracle.rapid(z, y, d, ua, us, 6.0, 2.0, want_dist=True)
    r1 = oracle.rapid(z / 2, y / 2, d, ua, us, 6.0, 1.0, want_dist=True)
    np.testing.assert_array_equal(r2.accept, r1.accept)
    np.testing.assert_array_equal(r2.token, r1.token)
    np.testing.assert_allclose(r2.emit_dist, r1.emit_dist, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(r2.phat_draft, r1.phat_draft, rtol=1e-12)


def _law_by_enumeration(z0, y0, eta, T, N=4000):
    """Emitted-token law at the first draft position, by exact enumeration over
    the draft token (weighted by q) and midpoint grids of the two uniforms,
    every decision taken by the oracle itself."""
    V = z0.size
    q = softmax(y0.astype(np.float64) / T)
    grid = ((np.arange(N) + 0.5) / N).astype(np.float32)
    z = np.stack([z0, z0]).astype(np.float32)
    y = np.stack([y0, y0]).astype(np.float32)
    # acceptance probability of each draft token
    acc = np.zeros(V)
    for x in range(V):
        r = oracle.rapid(np.repeat(z[None], N, 0), np.repeat(y[None], N, 0),
                         np.full((N, 1), x, np.int32), grid[:, None],
                         np.zeros((N, 2), np.float32), eta, T)
        acc[x] = r.accept[:, 0].mean()
    # draw after a rejection (an out-of-range draft forces it)
    r = oracle.rapid(np.repeat(z[None], N, 0), np.repeat(y[None], N, 0),
                     np.full((N, 1), V, np.int32), np.zeros((N, 1), np.float32),
                     np.stack([grid, np.zeros(N, np.float32)], 1), eta, T)
    draw = np.bincount(r.token, minlength=V) / N
    p_acc = float(np.sum(q * acc))
    return q * acc + (1.0 - p_acc) * draw, q


@pytest.mark.parametrize("case", range(4))
def test_sampler_law_equals_target(oracle_lib, case):
    """RAPID notes design 4 (and its key findings): with the adjusted residual
    the emitted token is distributed as the original target p wherever
    p >= min(q, phat) holds pointwise -- always at eta = 0 (textbook
    speculative sampling), and on the constructed rows for eta > 0."""
    rng = np.random.default_rng(100 + case)
    V = 6
    z0 = rng.normal(0, 1.5, V).astype(np.float32)
    if case == 0:
        eta, y0 = 0.0, rng.normal(0, 1.5, V).astype(np.float32)
    else:
        eta = [2.0, 5.0, 10.0][case - 1]
        y0 = (z0 + rng.normal(0, 0.3, V)).astype(np.float32)
    p = softmax(z0.astype(np.float64))
    ph = oracle.rapid_phat(z0.astype(np.float64), y0.astype(np.float64), eta, 1.0)
    q = softmax(y0.astype(np.float64))
    law, _ = _law_by_enumeration(z0, y0, eta, 1.0)
    if np.all(p >= np.minimum(q, ph) - 1e-15):
        np.testing.assert_allclose(law, p, atol=3e-3)
    else:
        # general law: min(q, phat) + (1 - sum min(q, phat)) * r / S
        m = np.minimum(q, ph)
        r = np.maximum(p - m, 0)
        np.testing.assert_allclose(law, m + (1 - m.sum()) * r / r.sum(), atol=3e-3)


def test_sampler_law_general_case(oracle_lib):
    """Where phat > p and q > p on some token the law is min(q, phat) +
    (1 - sum min(q, phat)) * r/S, no longer p; enumeration agrees."""
    z0 = np.array([0.0, 0.2, -0.4, 0.1, -1.0], np.float32)
    y0 = np.array([1.5, 0.0, -0.2, 0.0, -1.0], np.float32)
    eta = 8.0
    p = softmax(z0.astype(np.float64))
    ph = oracle.rapid_phat(z0.astype(np.float64), y0.astype(np.float64), eta, 1.0)
    q = softmax(y0.astype(np.float64))
    m = np.minimum(q, ph)
    assert np.any(p < m)  # the equality condition fails on this row
    law, _ = _law_by_enumeration(z0, y0, eta, 1.0)
    r = np.maximum(p - m, 0)
    np.testing.assert_allclose(law, m + (1 - m.sum()) * r / r.sum(), atol=3e-3)
    assert np.max(np.abs(law - p)) > 1e-2


# ------------------------------------------------- the ambiguity classifiers
# The parity rules exclude a request when one of these oracle outputs puts a
# decision within 1e-6 of its threshold, so each is pinned on rows built so
# that its value is known by hand.

def test_fused_gap_constructed(oracle_lib):
    """gap = top1 - top2 of the fp64 fused score t + beta*(a - b), counting a
    repeated maximum (gap 0, an exact tie), wherever the runner-up sits; inf
    for a one-token row.  Dyadic values: every score is exact."""
    V = 6
    zero = np.zeros(V, np.float32)
    cases = [  # (t, a, beta, gap, fused)
        ([0.0, 2.0, 1.5, 0.25, 1.0, -1.0], zero, 1.0, 0.5, 1),       # runner-up after the maximum
        ([1.5, 0.25, 2.0, 1.0, -1.0, 0.0], zero, 1.0, 0.5, 2),       # runner-up before it
        ([2.0, 0.0, 2.0, 1.0, -1.0, 0.0], zero, 1.0, 0.0, 0),        # repeated maximum: exact tie
        ([-3.0, -2.75, -3.5, -4.0, -5.0, -6.0], zero, 1.0, 0.25, 1),
        ([1.0, 1.25, 0.0, 0.0, 0.0, 0.0], [0.5, 0, 0, 0, 0, 0], 2.0, 0.75, 0),  # steered by delta = a - b
        ([1.0, 1.25, 0.0, 0.0, 0.0, 0.0], [0.5, 0, 0, 0, 0, 0], -2.0, 1.25, 1),  # negative beta
    ]
    for t_row, a_row, beta, gap, fused in cases:
        t = np.asarray(t_row, np.float32)[None, None]
        a = np.asarray(a_row, np.float32)[None, None]
        r = _asym(a, np.zeros_like(a), t, np.zeros((1, 0), np.int32), beta=beta)
        assert r.gap[0, 0] == gap and r.fused[0, 0] == fused
    one = np.zeros((1, 1, 1), np.float32)
    assert np.isinf(_asym(one, one, one, np.zeros((1, 0), np.int32)).gap[0, 0])


def test_acceptance_closeness_constructed(oracle_lib):
    """acc_rel = |u*q(x) - phat(x)| / max(u*q(x), phat(x)) at the draft.
    eta = 0 and a flat target: p = phat = 1/4 everywhere (no tail); the
    drafter holds all its mass on token 0 (q = 1).  The relative distance is
    taken against the larger side, and equality rejects."""
    z = np.zeros((2, 4), np.float32)
    y = np.array([[0.0, -np.inf, -np.inf, -np.inf]] * 2, np.float32)
    for u, rel, acc in [(0.125, 0.5, 1), (0.25, 0.0, 0), (0.5, 0.5, 0), (0.75, 2.0 / 3.0, 0)]:
        r = _rapid_one(z, y, [0], [u], [0.5, 0.5], 0.0, 1.0)
        assert r.q_draft[0, 0] == 1.0 and r.phat_draft[0, 0] == 0.25
        assert r.acc_rel[0, 0] == pytest.approx(rel, abs=1e-15)
        assert r.accept[0, 0] == acc
        # every token sits at the peak: ln 10 below the tail threshold's side
        assert r.tail_d_dist[0, 0] == pytest.approx(math.log(10.0), rel=1e-15)


def test_tail_distance_two_tokens(oracle_lib):
    """Two tokens, flat target (p = 1/2) and a drafter on token 0 (q = (1, 0)):
    zhat = z + eta*(q - p) = (eta/2, -eta/2), so token 1 sits eta below the
    peak and tail_d_dist there is |-eta - ln 0.1|.  At eta = 2 token 1 is
    above 10% of the peak (phat = 1/(1 + e^2)); at eta = 4 it is below and
    keeps p = 1/2."""
    z = np.zeros((2, 2), np.float32)
    y = np.array([[0.0, -np.inf]] * 2, np.float32)
    for eta, phat1 in [(2.0, 1.0 / (1.0 + math.exp(2.0))), (4.0, 0.5)]:
        r = _rapid_one(z, y, [1], [0.5], [0.5, 0.5], eta, 1.0)
        assert r.tail_d_dist[0, 0] == pytest.approx(abs(-eta - math.log(0.1)), rel=1e-12)
        assert r.phat_draft[0, 0] == pytest.approx(phat1, rel=1e-12)
        assert r.q_draft[0, 0] == 0.0 and r.acc_rel[0, 0] == 1.0 and r.accept[0, 0] == 1
        r0 = _rapid_one(z, y, [0], [0.5], [0.5, 0.5], eta, 1.0)
        ph0 = 1.0 / (1.0 + math.exp(-eta))
        assert r0.tail_d_dist[0, 0] == pytest.approx(-math.log(0.1), rel=1e-12)
        assert r0.phat_draft[0, 0] == pytest.approx(ph0, rel=1e-12)
        # u*q = 1/2 against the augmented phat (not p = 1/2): accepted
        assert r0.acc_rel[0, 0] == pytest.approx((ph0 - 0.5) / ph0, rel=1e-12) and r0.accept[0, 0] == 1


def test_tail_close_counts_emitting_row(oracle_lib):
    """tail_close counts the emitting row's tokens within 1e-6 of the tail
    threshold (zhat/T - Mhat = ln 0.1).  eta = 0, so zhat = z: two tokens at
    fp32(ln 0.1) (1e-8 from it), one 1e-3 away, the rest far below.  The
    drafter puts its mass on token 4, far in the target's tail, so the draft
    is rejected and row 0 is the emitting row; row 1 is flat."""
    l01 = math.log(0.1)
    z0 = [0.0, l01, l01, l01 + 1e-3, -20.0, -20.0, -20.0, -20.0]
    y0 = [-np.inf] * 8
    y0[4] = 0.0
    z = np.array([z0, [0.0] * 8], np.float32)
    y = np.array([y0, [0.0] * 8], np.float32)
    r = _rapid_one(z, y, [4], [0.5], [0.5, 0.5], 0.0, 1.0)
    assert r.accept_len[0] == 0
    assert r.tail_close[0] == 2
    # the same row as the second position, after an accepted first draft
    # (flat row, u = 0): row 1 emits and its tokens are the ones counted
    z2 = np.array([[0.0] * 8, z0, [0.0] * 8], np.float32)
    y2 = np.array([[0.0] * 8, y0, [0.0] * 8], np.float32)
    r2 = _rapid_one(z2, y2, [0, 4], [0.0, 0.5], [0.5, 0.5, 0.5], 0.0, 1.0)
    assert r2.accept_len[0] == 1
    assert r2.tail_close[0] == 2


def test_draw_slack_constructed(oracle_lib):
    """draw_slack = min(u*S - c_{k-1}, c_k - u*S) / S at the drawn token k.
    eta = 0, flat target (p = 1/4), drafter on token 0 (q = (1,0,0,0)), draft
    0 rejected at u = 1/2 (u*q = 1/2 > 1/4): the residual max(p - q, 0) is
    (0, 1/4, 1/4, 1/4), S = 3/4, cumulative (0, 1/4, 1/2, 3/4)."""
    z = np.zeros((2, 4), np.float32)
    y = np.array([[0.0, -np.inf, -np.inf, -np.inf]] * 2, np.float32)
    # fp32(1/3) is 1/3 + 1e-8: u*S lands 7.5e-9 past the end of token 1
    for us, tok, slack in [(0.5, 2, 1.0 / 6.0), (0.25, 1, 1.0 / 12.0), (0.625, 2, 1.0 / 24.0),
                           (1.0 / 3.0, 2, 0.0)]:
        us32 = float(np.float32(us))
        r = _rapid_one(z, y, [0], [0.5], [us32, 0.5], 0.0, 1.0)
        assert r.accept_len[0] == 0 and r.resid_S[0] == 0.75
        assert r.token[0] == tok
        assert r.draw_slack[0] == pytest.approx(slack, abs=1e-7)
