"""GPU parity of ``asym_verify_lmhead`` (AsymSpec from hidden states: the LM
heads' products on the matrix cores with the row statistics in their
epilogue) against the fp64 oracle (fp64 logits from the same bf16 inputs),
through the C ABI, on both of its paths: the JSD from stored (a, b) pairs
(full workspace) and from a and b formed a second time (minimal workspace,
no logit written).  The windows widen by the oracle's bound on the fp32
product-sum of each logit (oracle/parity.py, compare_lmhead)."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.parity import compare_lmhead

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[lmhead] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def _bf(vwl, x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).cuda()


def run_dev(vwl, x, beta, gamma, store_pairs=True):
    import torch
    d = torch.from_numpy(np.ascontiguousarray(x.draft)).cuda()
    out = vwl.asym_verify_lmhead(_bf(vwl, x.h_a), _bf(vwl, x.h_b), _bf(vwl, x.W_d), _bf(vwl, x.h_t),
                                 _bf(vwl, x.W_t), d, beta, gamma, store_pairs=store_pairs)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out._asdict().items()}


def check(vwl, x, beta=None, gamma=None, label=""):
    """Both paths against one oracle result; returns each path's outputs and
    report (stored pairs first) and the oracle's result."""
    beta = x.beta if beta is None else beta
    gamma = x.gamma if gamma is None else gamma
    lm = oracle.asym_lmhead(x.h_a, x.h_b, x.W_d, x.h_t, x.W_t, x.draft, beta, gamma)
    found = []
    for store in (True, False):
        _say("case %s B=%d K=%d V=%d Hd=%d Ht=%d beta=%g gamma=%g store_pairs=%s"
             % (label, x.B, x.K, x.V, x.Hd, x.Ht, beta, gamma, store))
        dev = run_dev(vwl, x, beta, gamma, store)
        rep = compare_lmhead(dev, lm, x.K, beta)
        _say("  " + str(rep))
        assert rep.ok, str(rep)
        assert dev["dev_err"][0] == 0
        found.append((dev, rep))
    return [f[0] for f in found], lm, [f[1] for f in found]


def test_small(vwl):
    x = W.gen_lmhead(3, 2, 1000, 128, seed=81)
    check(vwl, x, label="small")


@pytest.mark.parametrize("B,K,V,Hd", [(1, 0, 1, 64), (2, 1, 127, 64), (5, 4, 129, 192), (30, 2, 3001, 64),
                                      (23, 3, 20000, 128), (43, 2, 3001, 64), (50, 2, 1000, 128),
                                      (70, 2, 5000, 64), (129, 0, 700, 64)])
def test_shapes(vwl, B, K, V, Hd):
    """Row counts that are not multiples of the row tile (64 rows up to 128,
    192 rows past that: 129, 150, 210 rows), vocabularies below, at and past
    the 128-token tile, one token, no drafts."""
    x = W.gen_lmhead(B, K, max(V, 2), Hd, seed=82 + V + B) if V > 1 else None
    if x is None:  # one-token vocabulary: the generator needs two tokens to plant a spike
        x = W.gen_lmhead(B, K, 2, Hd, seed=82)
        x.W_d = np.ascontiguousarray(x.W_d[:1])
        x.W_t = np.ascontiguousarray(x.W_t[:1])
        x.draft[:] = 0
    check(vwl, x, label="shape")


def test_medium_vocabulary(vwl):
    """The Qwen3 vocabulary with small heads: many vocabulary ranges per row."""
    x = W.gen_lmhead(8, 2, 151936, 256, seed=83)
    devs, lm, reps = check(vwl, x, label="V=151936")
    assert all(rep.checked >= 6 for rep in reps)


def test_bench_shape(vwl):
    """B=64, K=2, V=151936, Hd=2560, Ht=5120: the shape the bench times.  At
    these head widths the worst-case product-sum bound is wide (a few 1e-2 on
    D), so more decisions fall in the windows; the deviations observed are
    near the fp32 rounding of the statistics."""
    x = W.lmhead_batched()
    for beta, gamma in ((1.0, 0.5), (0.0, 1.0)):
        devs, lm, reps = check(vwl, x, beta, gamma, label=x.name)
        for rep in reps:
            assert rep.checked >= 40
            assert rep.stats["D_max_abs"] < 1e-5


def test_bench_shape_exact_products(vwl):
    """The bench shape with signed power-of-two heads and hidden states: every
    fp32 product-sum is exact, so the device's logits equal the fp64 ones,
    the oracle's product bound is zero and the windows are the plain ones of
    the pass (D to 1e-5 relative); at most two requests may be excluded."""
    x = W.lmhead_dyadic()
    for beta, gamma in ((1.0, 0.5), (0.0, 1.0)):
        devs, lm, reps = check(vwl, x, beta, gamma, label=x.name)
        for e in (lm.err_a, lm.err_b, lm.err_t):
            assert np.all(e == 0.0)
        for rep in reps:
            assert rep.stats["D_window_max"] == 0.0
            assert rep.excluded <= 2
            assert rep.checked >= x.B - 2


def test_back_to_back_calls_reuse_the_workspace(vwl):
    """Calls of one shape share a workspace: the records, statistics, stored
    logit pairs and JSD partials one call leaves there must not reach the
    next (x, then y, then x again)."""
    x = W.gen_lmhead(6, 3, 9000, 128, seed=84)
    y = W.gen_lmhead(6, 3, 9000, 128, seed=85)
    lm = oracle.asym_lmhead(y.h_a, y.h_b, y.W_d, y.h_t, y.W_t, y.draft, y.beta, y.gamma)
    for store in (True, False):
        _say("case back-to-back B=6 K=3 V=9000 Hd=128 store_pairs=%s" % store)
        d1 = run_dev(vwl, x, x.beta, x.gamma, store)
        d2 = run_dev(vwl, y, y.beta, y.gamma, store)
        d3 = run_dev(vwl, x, x.beta, x.gamma, store)
        for k in d1:
            assert np.array_equal(d1[k], d3[k], equal_nan=True), k
        rep = compare_lmhead(d2, lm, y.K, y.beta)
        assert rep.ok, str(rep)


def test_bad_draft_ids(vwl):
    """A draft id outside [0, V) sets bit 0 of dev_err and rejects that draft;
    the other rows are unaffected."""
    x = W.gen_lmhead(4, 3, 3000, 64, seed=86)
    x.draft[0, 0] = -1
    x.draft[1, 2] = x.V
    _say("case bad drafts B=4 K=3 V=3000 Hd=64")
    dev = run_dev(vwl, x, 1.0, 0.5)
    assert dev["dev_err"][0] & 1
    assert dev["accept"][0, 0] == 0 and dev["accept"][1, 2] == 0
    assert dev["accept_len"][0] == 0 and dev["accept_len"][1] <= 2
    lm = oracle.asym_lmhead(x.h_a, x.h_b, x.W_d, x.h_t, x.W_t, x.draft, 1.0, 0.5)
    rep = compare_lmhead(dev, lm, x.K, 1.0)
    assert rep.ok, str(rep)


def test_workspace_sizes_pick_the_path(vwl):
    """A caller's workspace of the minimal size runs the path with no pair
    storage; one byte less is refused; the full size stores the pairs."""
    import torch
    lib = vwl.load_library()
    x = W.gen_lmhead(3, 2, 5000, 128, seed=87)
    full = lib.vwl_asym_lmhead_workspace_bytes(x.B, x.K, x.V, x.Hd, x.Ht)
    small = lib.vwl_asym_lmhead_workspace_min_bytes(x.B, x.K, x.V, x.Hd, x.Ht)
    assert 0 < small < full
    assert full - small >= 8 * x.B * (x.K + 1) * x.V
    lm = oracle.asym_lmhead(x.h_a, x.h_b, x.W_d, x.h_t, x.W_t, x.draft, x.beta, x.gamma)
    d = torch.from_numpy(np.ascontiguousarray(x.draft)).cuda()
    args = [_bf(vwl, v) for v in (x.h_a, x.h_b, x.W_d, x.h_t, x.W_t)] + [d, x.beta, x.gamma]
    for n in (small, full):
        _say("case workspace of %d bytes" % n)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        out = vwl.asym_verify_lmhead(*args, workspace=ws)
        torch.cuda.synchronize()
        dev = {k: v.cpu().numpy() for k, v in out._asdict().items()}
        rep = compare_lmhead(dev, lm, x.K, x.beta)
        assert rep.ok, str(rep)
    ws = torch.zeros(small - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        vwl.asym_verify_lmhead(*args, workspace=ws)
