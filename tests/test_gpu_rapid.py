"""GPU parity of ``rapid_verify`` against the fp64 oracle (RAPID notes, key
designs 2-4), through the C ABI, plus the law of the emitted token.

Rules (oracle/parity.py): accept flags, accept lengths and drawn tokens
exact outside the 1e-6 ambiguity windows (excluded and counted); phat and q
at the drafts within 1e-5 relative; the emitted distribution elementwise
within 1e-5 relative plus the rounding allowance of the residual's
subtractions."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.parity import compare_rapid

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[rapid] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def run_dev(vwl, x, eta=None, T=None, want=True):
    import torch
    eta = x.eta if eta is None else eta
    T = x.T if T is None else T
    z = vwl.to_device_logits(x.z, x.dtype)
    y = vwl.to_device_logits(x.y, x.dtype)
    d = torch.from_numpy(np.ascontiguousarray(x.draft)).cuda()
    ua = torch.from_numpy(np.ascontiguousarray(x.u_accept)).cuda()
    us = torch.from_numpy(np.ascontiguousarray(x.u_sample)).cuda()
    out = vwl.rapid_verify(z, y, d, ua, us, eta, T, want_probs=want, want_dist=want)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out._asdict().items()}


def check(vwl, x, eta=None, T=None, label="", min_checked=None):
    """Parity of one call.  Draws are excluded when u*S lies within 1e-6*S of
    an interval end; with V tokens each interval is about S/V wide, so the
    share of excluded draws grows with V (two or three of the sixteen at
    V = 128256).  At least min_checked requests must be checked (by
    default all but a quarter, and at least all but one)."""
    eta = x.eta if eta is None else eta
    if min_checked is None:
        min_checked = x.B - max(1, x.B // 4)
    T = x.T if T is None else T
    _say("case %s %s B=%d G=%d V=%d eta=%g T=%g" % (label, x.dtype, x.B, x.G, x.V, eta, T))
    dev = run_dev(vwl, x, eta, T)
    ora = oracle.rapid(x.z, x.y, x.draft, x.u_accept, x.u_sample, eta, T, x.dtype, want_dist=True)
    rep = compare_rapid(dev, ora, x.G)
    _say("  " + str(rep))
    assert rep.ok, str(rep)
    assert dev["dev_err"][0] == 0
    assert rep.checked >= min_checked
    return dev, ora, rep


@pytest.fixture(scope="module")
def c3():
    return W.rapid_c3()


@pytest.mark.parametrize("eta", W.C3_ETAS)
def test_rapid_b16_g10_v128256(vwl, c3, eta):
    check(vwl, c3, eta, 1.0, label="B16_G10_V128256", min_checked=13)


def test_rapid_upward_eta(vwl, c3):
    for eta in (40.0, 50.0):
        check(vwl, c3, eta, 1.0, label="upward", min_checked=13)


def test_rapid_eta_changes_decisions(vwl):
    """Full vocabulary with a +13 spike: the target's mass sits on few tokens,
    so the augmentation strength moves accept lengths and emitted tokens.
    Parity at each eta, and the oracle's decisions must differ between the
    unaugmented target and the augmented ones (else this case would not test
    the augmentation at this width)."""
    x = W.rapid_spiked()
    lens = {}
    for eta in (0.0, 5.0, 10.0, 20.0):
        dev, ora, rep = check(vwl, x, eta, 1.0, label="spiked", min_checked=13)
        lens[eta] = (np.asarray(ora.accept_len).copy(), np.asarray(ora.token).copy())
    for eta in (5.0, 10.0, 20.0):
        assert not np.array_equal(lens[eta][0], lens[0.0][0])
    assert not np.array_equal(lens[20.0][0], lens[5.0][0])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 5, 17, 1000, 1027, 4097, 9001])
@pytest.mark.parametrize("G", [0, 1, 3, 10])
def test_rapid_small_shapes(vwl, dtype, V, G):
    x = W.gen_rapid(4, G, V, dtype, seed=500 + V * 7 + G, eta=10.0)
    check(vwl, x, label="small")


@pytest.mark.parametrize("T", [0.5, 0.7, 2.0])
def test_rapid_temperature(vwl, T):
    x = W.gen_rapid(6, 5, 30011, "f32", seed=int(T * 100), eta=5.0, T=T)
    check(vwl, x, label="T")


@pytest.mark.parametrize("nv", [1, 2, 4, 8])
def test_rapid_every_plan(vwl, nv):
    x = W.gen_rapid(5, 4, 50000, "f32", seed=33, eta=20.0)
    try:
        vwl.set_plan_override("rapid", nv, 0)
        check(vwl, x, label="plan nv=%d" % nv)
    finally:
        vwl.set_plan_override("rapid", 0, 0)


def test_rapid_bad_inputs(vwl):
    x = W.gen_rapid(4, 3, 2000, "f32", seed=2, eta=5.0)
    x.draft[0, 0] = x.V + 5
    x.u_accept[1, 0] = 1.0
    x.u_sample[2, :] = np.nan
    dev = run_dev(vwl, x)
    assert dev["dev_err"][0] & 1 and dev["dev_err"][0] & 2
    ora = oracle.rapid(x.z, x.y, x.draft, x.u_accept, x.u_sample, x.eta, x.T)
    np.testing.assert_array_equal(dev["accept"], ora.accept)
    np.testing.assert_array_equal(dev["accept_len"], ora.accept_len)
    assert dev["accept"][0, 0] == 0 and dev["accept_len"][0] == 0


def test_rapid_deterministic(vwl, c3):
    d1 = run_dev(vwl, c3, 10.0, 1.0)
    d2 = run_dev(vwl, c3, 10.0, 1.0)
    for k in d1:
        if d1[k] is not None:
            assert np.array_equal(d1[k], d2[k]), k


def _law(vwl, z0, y0, eta, N, seed):
    """Emitted first-position token over N requests sharing one (z, y) pair:
    draft ~ q by Gumbel-max, fresh uniforms per request."""
    import torch
    rng = np.random.default_rng(seed)
    V = z0.size
    q = np.exp(y0.astype(np.float64) - y0.max())
    q /= q.sum()
    x = (np.argmax(y0[None, :].astype(np.float64) - np.log(-np.log(rng.random((N, V)))), axis=1)).astype(np.int32)
    z = torch.from_numpy(np.broadcast_to(np.stack([z0, z0]), (N, 2, V)).copy()).cuda()
    y = torch.from_numpy(np.broadcast_to(np.stack([y0, y0]), (N, 2, V)).copy()).cuda()
    ua = torch.from_numpy(W.uniforms_2p24(rng, (N, 1))).cuda()
    us = torch.from_numpy(W.uniforms_2p24(rng, (N, 2))).cuda()
    out = vwl.rapid_verify(z, y, torch.from_numpy(x[:, None]).cuda(), ua, us, eta, 1.0)
    torch.cuda.synchronize()
    acc = out.accept_len.cpu().numpy() >= 1
    tok = np.where(acc, x, out.token.cpu().numpy())
    return np.bincount(tok, minlength=V) / N


@pytest.mark.parametrize("eta", [0.0, 4.0])
def test_emitted_token_law(vwl, eta):
    """The emitted token follows p where p >= min(q, phat) pointwise (RAPID
    notes, key design 4); otherwise the general law min(q, phat) +
    (1 - sum min(q, phat)) * r/S.  Checked on 400k device draws."""
    from scipy.special import softmax
    rng = np.random.default_rng(7)
    V = 6
    z0 = rng.normal(0, 1.2, V).astype(np.float32)
    y0 = (z0 + rng.normal(0, 0.6, V)).astype(np.float32)
    N = 400000
    freq = _law(vwl, z0, y0, eta, N, 11)
    p = softmax(z0.astype(np.float64))
    q = softmax(y0.astype(np.float64))
    ph = oracle.rapid_phat(z0.astype(np.float64), y0.astype(np.float64), eta, 1.0)
    m = np.minimum(q, ph)
    r = np.maximum(p - m, 0)
    law = m + (1 - m.sum()) * r / r.sum()
    if eta == 0.0:
        np.testing.assert_allclose(law, p, atol=1e-12)
    sigma = np.sqrt(law * (1 - law) / N)
    _say("  law max |freq - law| / sigma = %.2f" % float(np.max(np.abs(freq - law) / sigma)))
    assert np.all(np.abs(freq - law) <= 5 * sigma + 1e-9)


def test_rapid_maximum_drafts(vwl):
    """G = 63, the largest number of drafts a call takes."""
    x = W.gen_rapid(2, 63, 3000, "f32", seed=41)
    check(vwl, x, 10.0, 1.0, label="G=63")


def test_rapid_largest_vocabulary(vwl):
    """V = VWL_RAPID_MAX_V (2^21), the tail's geometry limit (16 elements per
    thread, 512 workgroups per request)."""
    x = W.gen_rapid(1, 1, 1 << 21, "f32", seed=42)
    check(vwl, x, 10.0, 1.0, label="V=2^21")


def test_rapid_no_drafts(vwl):
    """G = 0: the bonus row alone; the token is drawn from p."""
    x = W.gen_rapid(3, 0, 5000, "f32", seed=43)
    dev, ora, rep = check(vwl, x, 10.0, 1.0, label="G=0")
    assert np.all(dev["accept_len"] == 0)


def test_rapid_back_to_back_calls_reuse_the_workspace(vwl):
    """Two calls of one shape on different inputs share the cached workspace:
    every published exchange word of the first call must be back to zero
    before the second (teams of more than 16 members, so members other than
    each row segment's first lane are covered)."""
    try:
        vwl.set_plan_override("rapid", 1, 0)
        for seed in (61, 62, 63):
            x = W.gen_rapid(3, 4, 50000, "f32", seed=seed, eta=8.0, T=0.8)
            check(vwl, x, label="reuse seed=%d" % seed)
    finally:
        vwl.set_plan_override("rapid", 0, 0)
