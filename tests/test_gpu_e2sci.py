"""GPU parity of ``e2sci_verify`` (E2-SCI notes, key design 3: per-position
JSD of drafter and target against the window threshold, the EWMA credit
state and the clamped next threshold) against the fp64 oracle, through the
C ABI.  Rules in oracle/parity.py (compare_e2sci)."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.parity import compare_e2sci

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[e2sci] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def _oracle_params(prm):
    return oracle.E2sciParams(alpha=prm.alpha, tau_credit=prm.tau_credit, T_base=prm.T_base,
                              T_min=prm.T_min, T_max=prm.T_max, ewma=prm.ewma, hysteresis=prm.hysteresis,
                              min_refresh=prm.min_refresh, delta=prm.delta, T_safe=prm.T_safe)


def run_dev(vwl, x, prm, T=None, r_hat=None, in_place=False, age=None):
    import torch
    y = vwl.to_device_logits(x.y, x.dtype)
    z = vwl.to_device_logits(x.z, x.dtype)
    Td = torch.from_numpy(np.ascontiguousarray(x.T if T is None else T, np.float32)).cuda()
    om = torch.from_numpy(np.ascontiguousarray(x.omega, np.float32)).cuda()
    rh = torch.from_numpy(np.ascontiguousarray(x.r_hat if r_hat is None else r_hat, np.float32)).cuda()
    ag = None if age is None else torch.from_numpy(np.ascontiguousarray(age, np.int32)).cuda()
    out = vwl.e2sci_verify(y, z, Td, om, rh, prm, age=ag, T_out=Td if in_place else None)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out._asdict().items()}


def check(vwl, x, prm=None, label="", T=None, r_hat=None, in_place=False, max_excluded=0, age=None):
    prm = prm if prm is not None else vwl.E2sciParams()
    T = x.T if T is None else np.asarray(T, np.float32)
    r_hat = x.r_hat if r_hat is None else np.asarray(r_hat, np.float32)
    _say("case %s %s B=%d W=%d V=%d" % (label, x.dtype, x.B, x.W, x.V))
    dev = run_dev(vwl, x, prm, T, r_hat, in_place, age)
    ora = oracle.e2sci(x.y, x.z, T, x.omega, r_hat, _oracle_params(prm), x.dtype, age=age)
    rep = compare_e2sci(dev, ora, T, identical=x.identical)
    _say("  " + str(rep))
    assert rep.ok, str(rep)
    assert dev["dev_err"][0] == 0
    assert rep.excluded <= max_excluded, "%d requests excluded" % rep.excluded
    return dev, ora, rep


def test_tiny_fp32(vwl):
    x = W.gen_e2sci(4, 4, 1024, "f32", seed=11, identical_frac=0.25)
    check(vwl, x, label="B4_W4_V1024")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 17, 1027, 151937])
@pytest.mark.parametrize("Wn", [1, 3, 8])
def test_small_and_ragged(vwl, dtype, V, Wn):
    x = W.gen_e2sci(3, Wn, V, dtype, seed=3000 + V + Wn, identical_frac=0.2)
    check(vwl, x, label="small")


def test_single_request_window(vwl):
    """B = 1, the pages' real-time batch; W = 8 drafts at V = 151936."""
    x = W.e2sci_single()
    dev, ora, rep = check(vwl, x, label=x.name)
    assert rep.checked + rep.excluded == 1


def test_batched(vwl):
    x = W.e2sci_batched()
    dev, ora, rep = check(vwl, x, label=x.name)
    assert rep.excluded <= 2
    assert 0 < ora.accept.mean() < 1


def test_thresholds_in_place_over_windows(vwl):
    """Five windows in a row with the credit state and the threshold carried
    on the device (T_out aliases T_in, r_hat updated in place); each window
    is checked against the oracle fed the same state."""
    import torch
    prm = vwl.E2sciParams(alpha=0.4, tau_credit=0.5, T_base=0.08, T_min=0.02, T_max=0.2, ewma=0.3)
    xs = [W.gen_e2sci(16, 4, 30000, "bf16", seed=500 + k, identical_frac=0.1) for k in range(5)]
    T = torch.from_numpy(xs[0].T.copy()).cuda()
    rh = torch.from_numpy(xs[0].r_hat.copy()).cuda()
    om = torch.from_numpy(xs[0].omega.copy()).cuda()
    for k, x in enumerate(xs):
        T_before = T.cpu().numpy().copy()
        r_before = rh.cpu().numpy().copy()
        out = vwl.e2sci_verify(vwl.to_device_logits(x.y, x.dtype), vwl.to_device_logits(x.z, x.dtype),
                               T, om, rh, prm, T_out=T)
        torch.cuda.synchronize()
        dev = {k2: (v.cpu().numpy() if v is not None else None) for k2, v in out._asdict().items()}
        assert out.T_next.data_ptr() == T.data_ptr()
        ora = oracle.e2sci(x.y, x.z, T_before, xs[0].omega, r_before, _oracle_params(prm), x.dtype)
        rep = compare_e2sci(dev, ora, T_before, identical=x.identical)
        _say("  window %d %s" % (k, rep))
        assert rep.ok, str(rep)


@pytest.mark.parametrize("nv", [1, 2, 4, 8])
def test_every_plan(vwl, nv):
    import torch
    x = W.gen_e2sci(6, 4, 40000, "bf16", seed=57, identical_frac=0.2)
    try:
        vwl.set_plan_override("asym", nv, 0)
        plan = vwl.e2sci_plan_info(6, 4, 40000, torch.bfloat16)
        assert plan["vec_per_thread"] == nv
        check(vwl, x, label="plan %s" % plan)
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_wide_team(vwl):
    """More than 128 members per row (one fp32 vector per thread)."""
    import torch
    x = W.gen_e2sci(2, 3, 151937, "f32", seed=92, identical_frac=0.2)
    try:
        vwl.set_plan_override("asym", 1, 0)
        plan = vwl.e2sci_plan_info(2, 3, 151937, torch.float32)
        assert plan["team"] > 128, plan
        check(vwl, x, label="wide team %s" % plan)
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_few_teams(vwl):
    x = W.gen_e2sci(16, 5, 20000, "f32", seed=79)
    try:
        vwl.set_plan_override("asym", 1, 3)
        check(vwl, x, label="3 teams")
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_inclusive_threshold_and_clamps(vwl):
    """Identical rows (D = 0) pass at T = 0; huge and tiny weights hit the
    clamps exactly."""
    x = W.gen_e2sci(8, 3, 5000, "f32", seed=80, identical_frac=0.0)
    x.y[:4] = x.z[:4]
    x.identical[:4] = True
    x.omega[:] = 1e4
    prm = vwl.E2sciParams(alpha=1.0, tau_credit=0.5, T_base=0.1, T_min=0.02, T_max=0.25, ewma=1.0)
    # the identical rows sit on the threshold (D = T = 0) and are ambiguous by
    # construction: the four are excluded by the rules and checked here directly
    dev, ora, rep = check(vwl, x, prm, T=np.zeros(8, np.float32), r_hat=np.zeros(8, np.float32), max_excluded=4)
    np.testing.assert_array_equal(dev["accept_len"][:4], 3)
    np.testing.assert_array_equal(dev["accept_len"][4:], 0)
    np.testing.assert_array_equal(dev["T_next"], np.float32([0.25] * 4 + [0.02] * 4))
    np.testing.assert_array_equal(dev["r_hat"], np.float32([1.0] * 4 + [0.0] * 4))


def test_stabilisers_batched(vwl):
    """The stabilisers on the batched workload: a dead band, a refresh
    interval of 3 windows with ages spread over 0..4, and a safety floor that
    some windows fall under; thresholds and counts match the oracle."""
    x = W.e2sci_batched()
    prm = vwl.E2sciParams(alpha=0.4, tau_credit=0.5, T_base=0.08, T_min=0.02, T_max=0.2, ewma=0.3,
                          hysteresis=0.01, min_refresh=3, delta=0.25, T_safe=0.03)
    age = (np.arange(x.B) % 5).astype(np.int32)
    dev, ora, rep = check(vwl, x, prm, label="stabilised " + x.name, age=age, max_excluded=2)
    p_acc = ora.accept_len / x.W
    assert np.any(p_acc < 0.25) and np.any((p_acc >= 0.25) & (age + 1 < 3))
    assert np.any(ora.age == 0) and np.any(ora.age > 0)
    ok = np.isfinite(ora.hyst_margin)
    assert np.any(ora.hyst_margin[ok] > 0) and np.any(ora.hyst_margin[ok] <= 0)


def test_stabilisers_over_windows(vwl):
    """Eight windows with the threshold, credit state and window count all
    carried on the device (T_out aliases T_in); each window is checked
    against the oracle fed the device's state before it."""
    import torch
    prm = vwl.E2sciParams(alpha=0.6, tau_credit=0.5, T_base=0.08, T_min=0.02, T_max=0.2, ewma=0.3,
                          hysteresis=0.005, min_refresh=2, delta=0.2, T_safe=0.03)
    xs = [W.gen_e2sci(16, 4, 30000, "bf16", seed=700 + k, identical_frac=0.1) for k in range(8)]
    T = torch.from_numpy(xs[0].T.copy()).cuda()
    rh = torch.from_numpy(xs[0].r_hat.copy()).cuda()
    om = torch.from_numpy(xs[0].omega.copy()).cuda()
    age = torch.zeros(16, dtype=torch.int32, device="cuda")
    held = 0
    for k, x in enumerate(xs):
        T_before = T.cpu().numpy().copy()
        r_before = rh.cpu().numpy().copy()
        a_before = age.cpu().numpy().copy()
        out = vwl.e2sci_verify(vwl.to_device_logits(x.y, x.dtype), vwl.to_device_logits(x.z, x.dtype),
                               T, om, rh, prm, age=age, T_out=T)
        torch.cuda.synchronize()
        dev = {k2: (v.cpu().numpy() if v is not None else None) for k2, v in out._asdict().items()}
        ora = oracle.e2sci(x.y, x.z, T_before, xs[0].omega, r_before, _oracle_params(prm), x.dtype,
                           age=a_before)
        rep = compare_e2sci(dev, ora, T_before, identical=x.identical)
        _say("  window %d %s" % (k, rep))
        assert rep.ok, str(rep)
        assert rep.excluded <= 1
        held += int(np.sum(ora.age > 0))
    assert held > 0


def test_preallocated_outputs(vwl):
    """``out=`` buffers: two calls in a row into the same buffers give the
    results of calls that allocate their own, and the returned tensors are
    the buffers themselves."""
    import torch
    x = W.gen_e2sci(3, 8, 20011, "bf16", seed=77)
    prm = vwl.E2sciParams()
    y = vwl.to_device_logits(x.y, x.dtype)
    z = vwl.to_device_logits(x.z, x.dtype)
    mk = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    buf = vwl.e2sci_out(x.B, x.W, "cuda")
    for _ in range(2):
        ref = vwl.e2sci_verify(y, z, mk(x.T), mk(x.omega), mk(x.r_hat), prm)
        got = vwl.e2sci_verify(y, z, mk(x.T), mk(x.omega), mk(x.r_hat), prm, out=buf)
        torch.cuda.synchronize()
        assert got.D.data_ptr() == buf.D.data_ptr() and got.dev_err.data_ptr() == buf.dev_err.data_ptr()
        for k in ("D", "accept", "accept_len", "T_next", "r_hat", "dev_err"):
            assert torch.equal(getattr(ref, k), getattr(got, k)), k
    with pytest.raises(ValueError):
        vwl.e2sci_verify(y, z, mk(x.T), mk(x.omega), mk(x.r_hat), prm, out=vwl.e2sci_out(x.B, x.W + 1, "cuda"))
