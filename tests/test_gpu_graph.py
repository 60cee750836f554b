"""Calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: every
replay must give the eager call's results bit for bit, with eager work and
synchronisations between the replays.  The library's kernels clear their own
counters (no memset nodes), so a replay needs no reset; the workspace is
passed explicitly, allocated before the capture."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[graph] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def _capture(fn):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def test_asym_single_request_replays(vwl):
    import torch
    x = W.single_asym()
    _say("asym B=%d K=%d V=%d %s" % (x.B, x.K, x.V, x.dtype))
    a, b, t = (vwl.to_device_logits(getattr(x, n), x.dtype) for n in "abt")
    d = torch.from_numpy(x.draft).cuda()
    ref = vwl.asym_verify(a, b, t, d, x.beta, x.gamma)
    torch.cuda.synchronize()
    ws = torch.zeros(vwl.workspace_bytes("asym", x.B, x.K, x.V, a.dtype), dtype=torch.uint8, device="cuda")
    out = vwl.asym_out(x.B, x.K, "cuda")
    g = _capture(lambda: vwl.asym_verify(a, b, t, d, x.beta, x.gamma, out=out, workspace=ws))
    other = W.tiny_asym()
    oa, ob, ot = (vwl.to_device_logits(getattr(other, n), other.dtype) for n in "abt")
    od = torch.from_numpy(other.draft).cuda()
    for rep in range(4):
        for f in out:
            f.fill_(-1 if f.dtype != torch.uint8 else 7)
        out.dev_err.zero_()
        g.replay()
        vwl.asym_verify(oa, ob, ot, od, other.beta, other.gamma)  # eager work between replays
        torch.cuda.synchronize()
        for k in ref._fields:
            assert torch.equal(getattr(ref, k), getattr(out, k)), (rep, k)
    _say("  4 replays identical to the eager call")


def test_e2sci_window_replays(vwl):
    """Four windows replayed from one graph carry the credit state on the
    device exactly as four eager calls do."""
    import torch
    x = W.e2sci_single()
    _say("e2sci B=%d W=%d V=%d %s" % (x.B, x.W, x.V, x.dtype))
    y = vwl.to_device_logits(x.y, x.dtype)
    z = vwl.to_device_logits(x.z, x.dtype)
    prm = vwl.E2sciParams()
    mk = lambda v: torch.from_numpy(np.ascontiguousarray(v, np.float32)).cuda()
    T, om, rh = mk(x.T), mk(x.omega), mk(x.r_hat)
    eager = []
    for _ in range(4):
        o = vwl.e2sci_verify(y, z, T, om, rh, prm, T_out=T)
        torch.cuda.synchronize()
        eager.append((o.D.clone(), o.accept.clone(), o.accept_len.clone(), T.clone(), rh.clone()))
    ws = torch.zeros(int(vwl.load_library().vwl_e2sci_workspace_bytes(x.B, x.W, x.V, vwl._dt(y))),
                     dtype=torch.uint8, device="cuda")
    out = vwl.e2sci_out(x.B, x.W, "cuda")
    T2, rh2 = mk(x.T), mk(x.r_hat)
    g = _capture(lambda: vwl.e2sci_verify(y, z, T2, om, rh2, prm, T_out=T2, out=out, workspace=ws))
    T2.copy_(mk(x.T))
    rh2.copy_(mk(x.r_hat))
    for rep in range(4):
        out.D.fill_(-1.0)
        out.accept.fill_(7)
        out.accept_len.fill_(-1)
        g.replay()
        vwl.e2sci_verify(y, z, mk(x.T), om, mk(x.r_hat), prm)  # eager work between replays
        torch.cuda.synchronize()
        got = (out.D, out.accept, out.accept_len, T2, rh2)
        for name, e, o in zip(("D", "accept", "accept_len", "T", "r_hat"), eager[rep], got):
            assert torch.equal(e, o), (rep, name)
    assert int(out.dev_err.item()) == 0
    _say("  4 chained windows identical to the eager calls")
