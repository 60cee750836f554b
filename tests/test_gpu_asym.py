"""GPU parity of ``asym_verify`` against the fp64 oracle (AsymSpec reading
notes, sections 4.1-4.2), through the C ABI.

Rules (oracle/parity.py): flags, accept lengths and tokens bit-exact outside
the 1e-6 ambiguity windows (excluded and counted; exact ties are never
excluded); D and gamma_eff within 1e-5 relative; D exactly 0 for identical
drafter rows."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.parity import compare_asym

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[asym] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def run_dev(vwl, x, beta=None, gamma=None):
    import torch
    beta = x.beta if beta is None else beta
    gamma = x.gamma if gamma is None else gamma
    a = vwl.to_device_logits(x.a, x.dtype)
    b = vwl.to_device_logits(x.b, x.dtype)
    t = vwl.to_device_logits(x.t, x.dtype)
    d = torch.from_numpy(np.ascontiguousarray(x.draft)).cuda()
    out = vwl.asym_verify(a, b, t, d, beta, gamma)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out._asdict().items()}


def check(vwl, x, beta=None, gamma=None, label="", max_excluded=0):
    """Parity of one call; at most max_excluded requests may fall in the
    ambiguity windows (the oracle's classifiers find none in these
    workloads, so the default is zero: a test cannot pass by excluding)."""
    beta = x.beta if beta is None else beta
    gamma = x.gamma if gamma is None else gamma
    _say("case %s %s B=%d K=%d V=%d beta=%g gamma=%g" % (label, x.dtype, x.B, x.K, x.V, beta, gamma))
    dev = run_dev(vwl, x, beta, gamma)
    ora = oracle.asym(x.a, x.b, x.t, x.draft, beta, gamma, x.dtype)
    rep = compare_asym(dev, ora, x.K, identical=np.all(x.a == x.b, axis=2))
    _say("  " + str(rep))
    assert rep.ok, str(rep)
    assert dev["dev_err"][0] == 0
    assert rep.excluded <= max_excluded, "%d requests excluded" % rep.excluded
    return dev, ora, rep


def test_tiny_fp32(vwl):
    check(vwl, W.tiny_asym(), label="B4_K2_V1024")


def test_single_request_fp32(vwl):
    x = W.single_asym()
    dev, ora, rep = check(vwl, x, label="B1_K2_V151936")
    assert rep.checked == 1


@pytest.fixture(scope="module")
def batched():
    return W.batched_asym()


@pytest.mark.parametrize("beta", W.C2_BETAS)
def test_batched_bf16_sweep(vwl, batched, beta):
    """The (beta, gamma) grid on the B=64, K=2, V=151936 bf16 inputs; D,
    gamma_eff and the flags must not move with beta."""
    prev = {}
    for gamma in W.C2_GAMMAS:
        dev, ora, rep = check(vwl, batched, beta, gamma, label="B64_K2_V151936")
        assert rep.excluded <= 2
        key = gamma
        if key in prev:
            for f in ("D", "gamma_eff", "accept", "accept_len"):
                assert np.array_equal(prev[key][f], dev[f])
        prev[key] = dev


def test_batched_beta_independence(vwl, batched):
    outs = [run_dev(vwl, batched, beta, 0.5) for beta in W.C2_BETAS]
    for o in outs[1:]:
        for f in ("D", "gamma_eff", "accept", "accept_len"):
            assert np.array_equal(o[f], outs[0][f]), f


def _standard_verification(vwl, x):
    """beta=0, gamma=1: fused == argmax t; fixed-threshold acceptance
    p_t(d) > p_b(d) implies CDA acceptance; equal where D == 0."""
    dev = run_dev(vwl, x, 0.0, 1.0)
    np.testing.assert_array_equal(dev["fused"], np.argmax(x.t, axis=2))
    ora = oracle.asym(x.a, x.b, x.t, x.draft, 0.0, 1.0, x.dtype)
    lt = ora.lse[..., 2]
    lb = ora.lse[..., 1]
    only_cda = 0
    for bi in range(x.B):
        for i in range(x.K):
            d = x.draft[bi, i]
            std_margin = (float(x.t[bi, i, d]) - lt[bi, i]) - (float(x.b[bi, i, d]) - lb[bi, i])
            if abs(std_margin) <= 1e-6 or abs(ora.margin[bi, i]) <= 1e-6:
                continue
            std = std_margin > 0
            if std:
                assert dev["accept"][bi, i] == 1
            if dev["D"][bi, i] == 0.0:
                assert bool(dev["accept"][bi, i]) == std
            if dev["accept"][bi, i] and not std:
                only_cda += 1
    return only_cda


def test_batched_standard_verification_point(vwl, batched):
    n = _standard_verification(vwl, batched)
    _say("  accepted by CDA only: %d" % n)


@pytest.fixture(scope="module")
def large():
    return W.large_asym()


def test_large_bf16(vwl, large):
    dev, ora, rep = check(vwl, large, label="B256_K4_V151936")
    assert np.all(dev["D"][large.identical] == 0.0)
    assert np.all(dev["gamma_eff"][large.identical] == np.float32(0.5))
    # planted ties: the lowest tied index wins
    for bi, i in np.argwhere(large.tie):
        s = large.t[bi, i].astype(np.float64) + (large.a[bi, i].astype(np.float64) - large.b[bi, i])
        assert dev["fused"][bi, i] == int(np.flatnonzero(s == s.max()).min())
    assert rep.stats["exact_ties"] >= large.tie.sum()


def test_large_standard_verification_point(vwl, large):
    n = _standard_verification(vwl, large)
    _say("  accepted by CDA only: %d" % n)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 5, 17, 1000, 1027])
@pytest.mark.parametrize("K", [0, 1, 2, 4, 10])
def test_small_shapes(vwl, dtype, V, K):
    x = W.gen_asym(3, K, V, dtype, seed=1000 + V * 13 + K, displaced_frac=0.3,
                   identical_frac=0.2 if 3 * (K + 1) >= 5 else 0.0)
    check(vwl, x, 1.0, 0.5, label="small")


@pytest.mark.parametrize("dtype,V", [("bf16", 151937), ("f32", 100003), ("bf16", 8191), ("f32", 65539)])
def test_ragged_rows(vwl, dtype, V):
    """Row starts off 16-byte boundaries (peeled head/tail) with multi-workgroup rows."""
    x = W.gen_asym(3, 2, V, dtype, seed=V, identical_frac=0.2, tie_frac=0.2)
    check(vwl, x, 1.0, 0.5, label="ragged")


@pytest.mark.parametrize("nv", [1, 2, 4, 8])
def test_every_plan(vwl, nv):
    """Each vectors-per-thread choice (different team sizes) reaches parity,
    with identical decisions."""
    x = W.gen_asym(6, 2, 40000, "bf16", seed=55, identical_frac=0.2, tie_frac=0.2)
    try:
        vwl.set_plan_override("asym", nv, 0)
        dev, ora, rep = check(vwl, x, 1.0, 0.5, label="plan nv=%d %s" % (nv, vwl.plan_info("asym", 6, 2, 40000, __import__("torch").bfloat16)))
        np.testing.assert_array_equal(dev["fused"], ora.fused)
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_wide_team(vwl):
    """More than 128 members per row (one fp32 vector per thread): every
    member-record loop of the combine and the finalize goes past the first
    two members per lane."""
    import torch
    x = W.gen_asym(2, 2, 151937, "f32", seed=91, identical_frac=0.2, tie_frac=0.2)
    try:
        vwl.set_plan_override("asym", 1, 0)
        plan = vwl.plan_info("asym", x.B, x.K, x.V, torch.float32)
        assert plan["team"] > 128, plan
        dev, ora, rep = check(vwl, x, 1.0, 0.5, label="wide team %s" % plan)
        np.testing.assert_array_equal(dev["fused"], ora.fused)
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_few_teams_many_rounds(vwl):
    """A capped team count forces many rows per team (counter reuse per row)."""
    x = W.gen_asym(16, 3, 20000, "f32", seed=77)
    try:
        vwl.set_plan_override("asym", 1, 3)
        check(vwl, x, 1.0, 0.5, label="3 teams")
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_deterministic_and_workspace_reuse(vwl):
    x = W.gen_asym(8, 2, 30000, "bf16", seed=8)
    y = W.gen_asym(8, 2, 30000, "bf16", seed=9)
    d1 = run_dev(vwl, x)
    d2 = run_dev(vwl, y)
    d3 = run_dev(vwl, x)
    for k in d1:
        assert np.array_equal(d1[k], d3[k]), k
    ora = oracle.asym(y.a, y.b, y.t, y.draft, y.beta, y.gamma, y.dtype)
    assert compare_asym(d2, ora, y.K, identical=np.all(y.a == y.b, axis=2)).ok


def test_bad_draft_ids(vwl):
    x = W.gen_asym(4, 3, 5000, "f32", seed=4)
    x.draft[0, 0] = -1
    x.draft[1, 2] = x.V
    dev = run_dev(vwl, x, 1.0, 0.0)
    assert dev["dev_err"][0] & 1
    assert dev["accept"][0, 0] == 0 and dev["accept"][1, 2] == 0
    assert dev["accept_len"][0] == 0 and dev["accept_len"][1] == 2
    ora = oracle.asym(x.a, x.b, x.t, x.draft, 1.0, 0.0, "f32")
    np.testing.assert_array_equal(dev["accept"], ora.accept)
    np.testing.assert_array_equal(dev["token"], ora.token)


def test_masked_logits(vwl):
    """-inf logits (masked tokens) have probability 0 in every softmax."""
    x = W.gen_asym(4, 2, 3000, "f32", seed=21)
    rng = np.random.default_rng(0)
    for arr in (x.a, x.b, x.t):
        m = rng.random(arr.shape) < 0.3
        arr[m] = -np.inf
    # keep every row non-empty and the drafts inside the support
    for arr in (x.a, x.b, x.t):
        arr[..., 0] = np.where(np.isfinite(arr[..., 0]), arr[..., 0], 0.0)
    x.draft[:] = np.argmax(x.a[:, :2], axis=2)
    check(vwl, x, 1.0, 0.5, label="masked")


def test_maximum_drafts(vwl):
    """K = 63, the largest number of drafts a call takes (64 rows per
    request), with identical drafter views so long accepted prefixes occur."""
    x = W.gen_asym(3, 63, 2000, "bf16", seed=31, identical_frac=0.5)
    dev, ora, rep = check(vwl, x, 1.0, 0.5, label="K=63")
    assert dev["accept"].shape == (3, 63)


def test_negative_beta_and_zero_gamma(vwl):
    """A negative fusion strength flips the context gain's sign (any finite
    beta is accepted); gamma = 0 accepts every draft with p_t(d) > 0."""
    x = W.gen_asym(6, 3, 9000, "f32", seed=32, identical_frac=0.2)
    check(vwl, x, -1.5, 0.5, label="beta=-1.5")
    dev, ora, rep = check(vwl, x, 1.0, 0.0, label="gamma=0")
    assert np.all(dev["accept"] == 1)


def test_single_element_rows(vwl):
    """V = 1: every softmax is the point mass, so D = 0 up to the rounding
    of the two single-element log-sum-exps (exactly 0 is promised only for
    bitwise-identical drafter rows), every fused token is 0, and the draft
    (token 0) passes for gamma < 1.  At gamma = 1 the margin is 0 up to that
    rounding: every draft sits in the ambiguity window and only parity
    outside it is required."""
    x = W.gen_asym(4, 3, 1, "f32", seed=33)
    dev, ora, rep = check(vwl, x, 1.0, 0.5, label="V=1")
    assert np.all(np.abs(dev["D"]) <= 1e-12) and np.all(dev["fused"] == 0) and np.all(dev["accept"] == 1)
    dev, ora, rep = check(vwl, x, 1.0, 1.0, label="V=1 gamma=1", max_excluded=4)
    assert rep.excluded == 4


def test_one_workspace_across_shapes(vwl):
    """One caller workspace, sized for the largest shape, reused by calls of
    three different shapes in a row (larger, smaller, larger again): every
    call leaves the workspace zero-filled, so each result stays within the
    parity rules."""
    import torch
    cases = [W.gen_asym(8, 4, 151936, "bf16", seed=W.SEED_BASE + 50),
             W.gen_asym(4, 2, 1024, "f32", seed=W.SEED_BASE + 51),
             W.gen_asym(3, 6, 50257, "f32", seed=W.SEED_BASE + 52)]
    need = max(vwl.workspace_bytes("asym", x.B, x.K, x.V, torch.bfloat16 if x.dtype == "bf16" else torch.float32)
               for x in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for x in cases * 2:
        _say("case shared-workspace %s B=%d K=%d V=%d" % (x.dtype, x.B, x.K, x.V))
        a = vwl.to_device_logits(x.a, x.dtype)
        b = vwl.to_device_logits(x.b, x.dtype)
        t = vwl.to_device_logits(x.t, x.dtype)
        d = torch.from_numpy(np.ascontiguousarray(x.draft)).cuda()
        out = vwl.asym_verify(a, b, t, d, x.beta, x.gamma, workspace=ws)
        torch.cuda.synchronize()
        dev = {k: v.cpu().numpy() for k, v in out._asdict().items()}
        ora = oracle.asym(x.a, x.b, x.t, x.draft, x.beta, x.gamma, x.dtype)
        rep = compare_asym(dev, ora, x.K, identical=np.all(x.a == x.b, axis=2))
        _say("  " + str(rep))
        assert rep.ok and dev["dev_err"][0] == 0, str(rep)
        assert int(ws.count_nonzero()) == 0, "the call left workspace bytes set"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wide_disagreement(vwl, dtype):
    """Drafter rows whose log-probability ratio x = ln p - ln q spreads over
    [-7, 7]: the divergence pass evaluates |x| < 4 by its polynomial and
    recomputes vectors holding a larger |x| exactly, so every row mixes both
    paths, with elements on both sides of the switch; D within 1e-5 relative."""
    x = W.gen_asym(6, 2, 40000, dtype, seed=34, identical_frac=0.0)
    rng = np.random.default_rng(34)
    shift = rng.uniform(-7.0, 7.0, size=x.a.shape)
    x.b = W._to_dtype(x.a.astype(np.float64) + shift, dtype)
    dev, ora, rep = check(vwl, x, label="wide disagreement")
    assert np.all(ora.D > 0.05)


def test_beside_a_running_kernel(vwl):
    """asym_verify launched while a chain of large GEMMs runs on a second
    stream of the same (default) priority.  The row kernel's workgroups then
    start only as the GEMM's workgroups retire, so its teams fill gradually;
    tickets are taken in start order, so every started member's team has all
    its earlier members started, and a partial team waits only for members
    that start once some workgroup retires.  Parity, dev_err == 0, and the
    GEMM's result is unaffected."""
    import torch
    x = W.batched_asym()
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    A = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
    Bm = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
    ref = (A[:64].float() @ Bm.float()).cpu()
    torch.cuda.synchronize()
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        outs = [A @ Bm for _ in range(6)]
    _say("GEMM chain queued on a second stream")
    dev, ora, rep = check(vwl, x, label="beside a GEMM chain")
    torch.cuda.synchronize()
    assert rep.checked == x.B
    for o in outs:
        np.testing.assert_allclose(o[:64].float().cpu().numpy(), ref.numpy(), rtol=2e-2, atol=2.0)
