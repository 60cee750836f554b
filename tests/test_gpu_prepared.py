"""Prepared calls (``prepare=True``): the arguments are checked and
marshalled once; each invocation must give what the ordinary call gives on
the same memory, also after the inputs are refilled in place."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[prepared] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def _equal(x, y, fields):
    import torch
    for k in fields:
        a, b = getattr(x, k), getattr(y, k)
        if a is None and b is None:
            continue
        assert torch.equal(a, b), k


def test_asym_prepared(vwl):
    import torch
    x1, x2 = W.gen_asym(3, 2, 20011, "bf16", seed=71), W.gen_asym(3, 2, 20011, "bf16", seed=72)
    _say("asym B=3 K=2 V=20011 bf16")
    a, b, t = (vwl.to_device_logits(getattr(x1, n), x1.dtype) for n in "abt")
    d = torch.from_numpy(x1.draft).cuda()
    call = vwl.asym_verify(a, b, t, d, 1.0, 0.5, out=vwl.asym_out(3, 2, "cuda"), prepare=True)
    for x in (x1, x2, x1):
        for dst, n in zip((a, b, t), "abt"):
            dst.copy_(vwl.to_device_logits(getattr(x, n), x.dtype))
        d.copy_(torch.from_numpy(x.draft))
        got = call()
        ref = vwl.asym_verify(a, b, t, d, 1.0, 0.5)
        torch.cuda.synchronize()
        _equal(got, ref, ("D", "gamma_eff", "accept", "fused", "accept_len", "token", "dev_err"))


def test_e2sci_prepared(vwl):
    import torch
    x = W.gen_e2sci(2, 8, 30011, "bf16", seed=73)
    _say("e2sci B=2 W=8 V=30011 bf16")
    y, z = vwl.to_device_logits(x.y, x.dtype), vwl.to_device_logits(x.z, x.dtype)
    mk = lambda v: torch.from_numpy(np.ascontiguousarray(v, np.float32)).cuda()
    prm = vwl.E2sciParams()
    T1, r1, om = mk(x.T), mk(x.r_hat), mk(x.omega)
    T2, r2 = mk(x.T), mk(x.r_hat)
    call = vwl.e2sci_verify(y, z, T1, om, r1, prm, T_out=T1, out=vwl.e2sci_out(2, 8, "cuda"), prepare=True)
    for _ in range(3): # windows chained on the device, both ways
        got = call()
        ref = vwl.e2sci_verify(y, z, T2, om, r2, prm, T_out=T2)
        torch.cuda.synchronize()
        _equal(got, ref, ("D", "accept", "accept_len", "T_next", "r_hat", "dev_err"))


def test_rapid_prepared(vwl):
    import torch
    x = W.gen_rapid(3, 4, 20011, "f32", seed=74, eta=6.0)
    _say("rapid B=3 G=4 V=20011 f32")
    z, y = vwl.to_device_logits(x.z, x.dtype), vwl.to_device_logits(x.y, x.dtype)
    d = torch.from_numpy(x.draft).cuda()
    ua, us = torch.from_numpy(x.u_accept).cuda(), torch.from_numpy(x.u_sample).cuda()
    call = vwl.rapid_verify(z, y, d, ua, us, x.eta, x.T, out=vwl.rapid_out(3, 4, x.V, "cuda", True, True),
                            prepare=True)
    for _ in range(2):
        got = call()
        ref = vwl.rapid_verify(z, y, d, ua, us, x.eta, x.T, want_probs=True, want_dist=True)
        torch.cuda.synchronize()
        _equal(got, ref, ("accept", "accept_len", "token", "p_hat_draft", "q_draft", "emit_dist", "dev_err"))
