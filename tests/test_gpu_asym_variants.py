"""GPU parity of ``asym_verify_variant`` (the AsymSpec notes' mechanism
ablation: fusion source delta = a - b, a or t - b; the CDA threshold or a
fixed gamma) against the fp64 oracle, through the C ABI.

Same rules as the default pass (oracle/parity.py); under the fixed gate the
device reports no divergence (D is NaN) and gamma_eff is gamma exactly."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.parity import compare_asym

pytestmark = pytest.mark.gpu

VARIANTS = [(d, g) for g in ("cda", "fixed") for d in ("a-b", "a", "t-b")]


def _say(msg):
    print("[asym-variant] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def run_dev(vwl, x, beta, gamma, delta, gate, drop_a=False):
    import torch
    a = None if drop_a else vwl.to_device_logits(x.a, x.dtype)
    b = vwl.to_device_logits(x.b, x.dtype)
    t = vwl.to_device_logits(x.t, x.dtype)
    d = torch.from_numpy(np.ascontiguousarray(x.draft)).cuda()
    out = vwl.asym_verify_variant(a, b, t, d, beta, gamma, delta, gate)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out._asdict().items()}


def check(vwl, x, delta, gate, beta=1.0, gamma=0.5, label="", drop_a=False, max_excluded=0):
    _say("case %s delta=%s gate=%s %s B=%d K=%d V=%d beta=%g gamma=%g" % (
        label, delta, gate, x.dtype, x.B, x.K, x.V, beta, gamma))
    dev = run_dev(vwl, x, beta, gamma, delta, gate, drop_a)
    ora = oracle.asym(x.a, x.b, x.t, x.draft, beta, gamma, x.dtype, delta=delta, gate=gate)
    rep = compare_asym(dev, ora, x.K, identical=np.all(x.a == x.b, axis=2), gate=gate)
    _say("  " + str(rep))
    assert rep.ok, str(rep)
    assert dev["dev_err"][0] == 0
    assert rep.excluded <= max_excluded, "%d requests excluded" % rep.excluded
    return dev, ora, rep


@pytest.mark.parametrize("delta,gate", VARIANTS)
def test_tiny_fp32(vwl, delta, gate):
    check(vwl, W.tiny_asym(), delta, gate, label="B4_K2_V1024")


@pytest.mark.parametrize("delta,gate", VARIANTS)
@pytest.mark.parametrize("dtype,V", [("f32", 1), ("bf16", 3), ("f32", 17), ("bf16", 1027), ("bf16", 151937)])
def test_small_and_ragged(vwl, delta, gate, dtype, V):
    x = W.gen_asym(3, 2, V, dtype, seed=2000 + V, displaced_frac=0.3, identical_frac=0.2,
                   tie_frac=0.2 if V > 16 else 0.0)
    check(vwl, x, delta, gate, 1.0, 0.5, label="small")


@pytest.fixture(scope="module")
def batched():
    return W.batched_asym()


@pytest.mark.parametrize("delta,gate", VARIANTS)
def test_batched_bf16(vwl, batched, delta, gate):
    """B=64, K=2, V=151936 bf16 at three (beta, gamma) points."""
    for beta, gamma in ((1.0, 0.5), (2.0, 0.4), (0.0, 1.0)):
        dev, ora, rep = check(vwl, batched, delta, gate, beta, gamma, label="B64_K2_V151936")
        assert rep.excluded <= 2


@pytest.fixture(scope="module")
def large():
    return W.large_asym()


@pytest.mark.parametrize("delta,gate", VARIANTS)
def test_large_bf16(vwl, large, delta, gate):
    """B=256, K=4, V=151936 bf16 with the identical-row and planted-tie
    structure; the planted ties of the default score resolve to the lowest
    index under every source (the copied column repeats a, b and t)."""
    dev, ora, rep = check(vwl, large, delta, gate, label="B256_K4_V151936")
    if gate == "cda":
        assert np.all(dev["D"][large.identical] == 0.0)
    for bi, i in np.argwhere(large.tie):
        a64 = large.a[bi, i].astype(np.float64)
        b64 = large.b[bi, i].astype(np.float64)
        t64 = large.t[bi, i].astype(np.float64)
        delta_v = {"a-b": a64 - b64, "a": a64, "t-b": t64 - b64}[delta]
        s = t64 + delta_v
        top = np.flatnonzero(s == s.max())
        if len(top) > 1:
            assert dev["fused"][bi, i] == int(top.min())


def test_default_variant_is_asym_verify(vwl, batched):
    """asym_verify_variant(a - b, CDA) returns asym_verify's bits."""
    import torch
    a = vwl.to_device_logits(batched.a, batched.dtype)
    b = vwl.to_device_logits(batched.b, batched.dtype)
    t = vwl.to_device_logits(batched.t, batched.dtype)
    d = torch.from_numpy(np.ascontiguousarray(batched.draft)).cuda()
    o1 = vwl.asym_verify(a, b, t, d, 1.0, 0.5)
    o1 = {k: v.cpu().numpy() for k, v in o1._asdict().items()}
    o2 = vwl.asym_verify_variant(a, b, t, d, 1.0, 0.5, "a-b", "cda")
    o2 = {k: v.cpu().numpy() for k, v in o2._asdict().items()}
    for k in o1:
        assert np.array_equal(o1[k], o2[k]), k


def test_two_model_difference_without_a(vwl, batched):
    """The fixed gate with delta = t - b never reads a: a null a gives the
    same bits as a real one."""
    with_a = run_dev(vwl, batched, 1.0, 0.5, "t-b", "fixed")
    without = run_dev(vwl, batched, 1.0, 0.5, "t-b", "fixed", drop_a=True)
    for k in with_a:
        assert np.array_equal(with_a[k], without[k], equal_nan=(k == "D")), k
    check(vwl, batched, "t-b", "fixed", label="a=null", drop_a=True)


@pytest.mark.parametrize("nv", [1, 2, 4, 8])
@pytest.mark.parametrize("delta", ["a", "t-b"])
def test_every_plan_fixed_gate(vwl, nv, delta):
    """Each vectors-per-thread choice of the single-pass (fixed-gate) kernel."""
    import torch
    x = W.gen_asym(6, 2, 40000, "bf16", seed=56, identical_frac=0.2, tie_frac=0.2)
    try:
        vwl.set_plan_override("asym", nv, 0)
        plan = vwl.asym_plan_info(6, 2, 40000, torch.bfloat16, delta, "fixed")
        assert plan["vec_per_thread"] == nv
        dev, ora, rep = check(vwl, x, delta, "fixed", label="plan %s" % plan)
        np.testing.assert_array_equal(dev["fused"], ora.fused)
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_fixed_gate_few_teams(vwl):
    """Many rows per team through the single-pass loop."""
    x = W.gen_asym(16, 3, 20000, "f32", seed=78)
    try:
        vwl.set_plan_override("asym", 1, 3)
        check(vwl, x, "a-b", "fixed", label="3 teams")
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_gate_relation_on_device(vwl, batched):
    """Every draft the fixed gate accepts, CDA accepts too (D >= 0)."""
    f = run_dev(vwl, batched, 1.0, 0.5, "a-b", "fixed")
    c = run_dev(vwl, batched, 1.0, 0.5, "a-b", "cda")
    assert np.all(c["accept"] >= f["accept"])
    np.testing.assert_array_equal(c["fused"], f["fused"])
