"""``asym_verify_noalloc`` (the entry point without a workspace argument,
whose workspace is the library's static per-device scratch) against
``asym_verify`` with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller input, each bit-identical to the workspace
call and within the oracle's parity rules."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.parity import compare_asym

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[noalloc] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def _both(vwl, x):
    import torch
    a = vwl.to_device_logits(x.a, x.dtype)
    b = vwl.to_device_logits(x.b, x.dtype)
    t = vwl.to_device_logits(x.t, x.dtype)
    d = torch.from_numpy(np.ascontiguousarray(x.draft)).cuda()
    ref = vwl.asym_verify(a, b, t, d, x.beta, x.gamma)
    got = vwl.asym_verify_noalloc(a, b, t, d, x.beta, x.gamma)
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in ref._asdict().items()},
            {k: v.cpu().numpy() for k, v in got._asdict().items()})


def test_noalloc_matches_workspace_call_twice(vwl):
    cases = [W.gen_asym(8, 4, 151936, "bf16", seed=W.SEED_BASE + 40),  # larger first
             W.gen_asym(4, 2, 1024, "f32", seed=W.SEED_BASE + 41)]     # then smaller
    for x in cases:
        _say("case %s B=%d K=%d V=%d" % (x.dtype, x.B, x.K, x.V))
        ref, got = _both(vwl, x)
        for k in ref:
            assert np.array_equal(ref[k], got[k], equal_nan=True), k
        assert got["dev_err"][0] == 0
        ora = oracle.asym(x.a, x.b, x.t, x.draft, x.beta, x.gamma, x.dtype)
        rep = compare_asym(got, ora, x.K, identical=np.all(x.a == x.b, axis=2))
        _say("  " + str(rep))
        assert rep.ok and rep.checked >= x.B - 1, str(rep)


def test_noalloc_rejects_oversized_shape(vwl):
    import torch
    lib = vwl.load_library()
    # 3400 bf16 rows of V = 151936 need more than the 16 MiB scratch; the
    # size check comes before any pointer is used
    code = lib.asym_verify_noalloc(None, None, None, None, 3400, 0, 151936, vwl.VWL_BF16, 1.0, 0.5,
                                   None, None, None, None, None, None, None,
                                   torch.cuda.current_stream().cuda_stream)
    assert code == 8
    assert "scratch" in lib.vwl_status_string(code).decode()
