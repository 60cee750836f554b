"""GPU parity of ``asym_verify_xfam`` (AsymSpec across model families: the
drafter's gain reaches the verifier through a vocabulary alignment, generation
restricted to the paired tokens) against the fp64 oracle, through the C ABI.
Rules as for asym_verify (oracle/parity.py)."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.parity import compare_asym

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[xfam] " + msg, flush=True)


@pytest.fixture(scope="module")
def vwl():
    import vocab_wide_logit_amd as m
    m.load_library()
    return m


def run_dev(vwl, x, beta=None, gamma=None, t=None, vmap=None, draft=None):
    import torch
    beta = x.beta if beta is None else beta
    gamma = x.gamma if gamma is None else gamma
    a = vwl.to_device_logits(x.a, x.dtype)
    b = vwl.to_device_logits(x.b, x.dtype)
    tt = vwl.to_device_logits(x.t if t is None else t, x.dtype)
    vm = torch.from_numpy(np.ascontiguousarray(x.vmap if vmap is None else vmap, np.int32)).cuda()
    d = torch.from_numpy(np.ascontiguousarray(x.draft if draft is None else draft, np.int32)).cuda()
    out = vwl.asym_verify_xfam(a, b, tt, vm, d, beta, gamma)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out._asdict().items()}


def check(vwl, x, beta=None, gamma=None, label="", t=None, vmap=None, draft=None, dev_err=0, max_excluded=0):
    beta = x.beta if beta is None else beta
    gamma = x.gamma if gamma is None else gamma
    t = x.t if t is None else t
    vmap = x.vmap if vmap is None else vmap
    draft = x.draft if draft is None else draft
    _say("case %s %s B=%d K=%d Vd=%d Vt=%d pairs=%d" % (label, x.dtype, x.B, x.K, x.Vd, x.Vt,
                                                      int((np.asarray(vmap) >= 0).sum())))
    dev = run_dev(vwl, x, beta, gamma, t, vmap, draft)
    ora = oracle.asym_xfam(x.a, x.b, t, vmap, draft, beta, gamma, x.dtype)
    rep = compare_asym(dev, ora, x.K, identical=np.all(x.a == x.b, axis=2))
    _say("  " + str(rep))
    assert rep.ok, str(rep)
    assert dev["dev_err"][0] == dev_err
    assert rep.excluded <= max_excluded, "%d requests excluded" % rep.excluded
    return dev, ora, rep


def test_tiny_fp32(vwl):
    check(vwl, W.gen_xfam(4, 2, 1024, 900, 700, "f32", seed=21), label="tiny")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Vd,Vt,n", [(1, 1, 1), (7, 5, 3), (1027, 4099, 900), (5000, 4096, 3000),
                                     (151937, 128257, 100000)])
def test_shapes(vwl, dtype, Vd, Vt, n):
    """Ragged vocabularies on both sides, a verifier larger than the drafter,
    exact multiples of the verifier chunk, tiny rows."""
    x = W.gen_xfam(3, 2, Vd, Vt, max(0, n - min(16, Vd, Vt)), dtype, seed=4000 + Vd + Vt,
                   n_special=min(16, Vd, Vt))
    check(vwl, x, label="shape")


def test_batched_qwen_to_llama(vwl):
    """B=64, K=2: Qwen-family drafter (151936), Llama-family verifier
    (128256), 109,566 shared tokens plus special pairs, bf16."""
    x = W.xfam_batched()
    for beta, gamma in ((1.0, 0.5), (2.0, 0.4), (0.0, 1.0)):
        dev, ora, rep = check(vwl, x, beta, gamma, label=x.name)
        assert rep.excluded <= 2


def test_identity_alignment_matches_asym_verify(vwl):
    """One vocabulary, identity alignment: the same bits as asym_verify."""
    import torch
    x = W.gen_asym(8, 3, 30011, "bf16", seed=22, identical_frac=0.2, tie_frac=0.2)
    a = vwl.to_device_logits(x.a, x.dtype)
    b = vwl.to_device_logits(x.b, x.dtype)
    t = vwl.to_device_logits(x.t, x.dtype)
    d = torch.from_numpy(np.ascontiguousarray(x.draft)).cuda()
    vm = torch.arange(x.V, dtype=torch.int32, device="cuda")
    o1 = {k: v.cpu().numpy() for k, v in vwl.asym_verify(a, b, t, d, 1.0, 0.5)._asdict().items()}
    o2 = {k: v.cpu().numpy() for k, v in vwl.asym_verify_xfam(a, b, t, vm, d, 1.0, 0.5)._asdict().items()}
    for k in ("fused", "accept", "accept_len", "token", "D", "gamma_eff"):
        assert np.array_equal(o1[k], o2[k]), k


def test_unpaired_and_bad_entries(vwl):
    """A huge logit on an unpaired verifier token is never emitted; a draft on
    an unpaired token is rejected; an alignment entry outside [-1, Vd) counts
    as unpaired and sets the map bit; a draft id outside [0, Vt) sets the
    draft bit; no pair at all gives fused = -1."""
    x = W.gen_xfam(4, 2, 3000, 2800, 2000, "f32", seed=23)
    free = np.flatnonzero(x.vmap < 0)
    t = x.t.copy()
    t[:, :, free[0]] = 1e4
    d = x.draft.copy()
    d[0, 0] = free[1]
    dev, ora, rep = check(vwl, x, t=t, draft=d, label="unpaired")
    assert np.all(x.vmap[dev["fused"]] >= 0) and dev["accept"][0, 0] == 0
    bad = x.vmap.copy()
    bad[free[2]] = x.Vd + 5
    bad[free[3]] = -7
    check(vwl, x, vmap=bad, label="bad entries", dev_err=8)
    d2 = x.draft.copy()
    d2[1, 1] = x.Vt
    dev, _, _ = check(vwl, x, draft=d2, label="draft out of range", dev_err=1)
    assert dev["accept"][1, 1] == 0
    # no pair: every fused score is -inf, the rules mark each request ambiguous
    # and the defined result (-1 everywhere) is checked directly
    dev, _, _ = check(vwl, x, vmap=np.full(x.Vt, -1, np.int32), label="no pairs", max_excluded=4)
    assert np.all(dev["fused"] == -1) and np.all(dev["token"] == -1)


@pytest.mark.parametrize("nv", [1, 2, 4, 8])
def test_every_plan(vwl, nv):
    x = W.gen_xfam(6, 2, 40000, 33000, 25000, "bf16", seed=24)
    try:
        vwl.set_plan_override("asym", nv, 0)
        check(vwl, x, label="plan nv=%d" % nv)
    finally:
        vwl.set_plan_override("asym", 0, 0)


def test_repeated_drafter_ids_and_flag_reset(vwl):
    """A map that pairs some drafter tokens with several verifier tokens meets
    the pairs in verifier order (the flag set by the inversion); the next call
    with a one-to-one map meets them in drafter order again, so the flag and
    the inverse map were cleared."""
    x = W.gen_xfam(4, 2, 3000, 2800, 2000, "bf16", seed=25)
    vm = x.vmap.copy()
    paired = np.flatnonzero(vm >= 0)
    rep = paired[1::7]
    vm[rep] = vm[paired[0::7][:len(rep)]]
    assert len(np.unique(vm[vm >= 0])) < int((vm >= 0).sum())
    check(vwl, x, vmap=vm, label="repeated drafter ids")
    check(vwl, x, label="one-to-one again")
    check(vwl, x, vmap=vm, label="repeated drafter ids again")


def test_equal_scores_resolve_to_lowest_verifier_id(vwl):
    """Two pairs with equal fused scores, the lower verifier id paired with
    the higher drafter id: the drafter-order pass meets the higher verifier id
    first and must still report the lower one."""
    x = W.gen_xfam(4, 2, 3000, 2800, 2000, "f32", seed=26)
    paired = np.flatnonzero(x.vmap >= 0)
    v_lo = v_hi = None
    for i in range(len(paired) - 1):
        for j in range(i + 1, min(i + 50, len(paired))):
            if x.vmap[paired[i]] > x.vmap[paired[j]]:
                v_lo, v_hi = int(paired[i]), int(paired[j])
                break
        if v_lo is not None:
            break
    assert v_lo is not None and v_lo < v_hi
    d_lo, d_hi = int(x.vmap[v_lo]), int(x.vmap[v_hi])
    assert d_lo > d_hi
    t = x.t.copy()
    t[:, :, v_lo] = 60.0
    t[:, :, v_hi] = 60.0
    x.a[:, :, d_lo] = x.a[:, :, d_hi]
    x.b[:, :, d_lo] = x.b[:, :, d_hi]
    dev, ora, rep = check(vwl, x, t=t, label="planted tie")
    assert np.all(dev["fused"] == v_lo)
    assert np.all(ora.fused == v_lo)


def _with_xfam(vwl, general=False, segs=0):
    class _Ctx:
        def __enter__(self):
            vwl.set_xfam_override(general, segs)

        def __exit__(self, *exc):
            vwl.set_xfam_override(False, 0)
    return _Ctx()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Vd,Vt,n", [(8, 8, 6), (4096, 40000, 3000), (65544, 65544, 50000),
                                     (151936, 128256, 100000)])
def test_staged_and_general_passes(vwl, dtype, Vd, Vt, n):
    """Vocabularies of whole 16-byte vectors take the staged verifier pass
    (the verifier row in LDS parts: one part, two for bf16 past 64K tokens,
    four for fp32 at 128K); each segment count and the general pass (a and b
    gathered through the map) give the oracle's results."""
    x = W.gen_xfam(3, 2, Vd, Vt, max(0, n - min(16, Vd, Vt)), dtype, seed=5000 + Vd + Vt,
                   n_special=min(16, Vd, Vt))
    for general, segs in ((False, 0), (False, 1), (False, 3), (False, 16), (True, 0)):
        with _with_xfam(vwl, general, segs):
            check(vwl, x, label="general" if general else "staged segs=%d" % segs)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeated_drafter_ids_both_passes(vwl, dtype):
    """Repeated drafter ids over several verifier parts (bf16 and fp32 rows
    past one part), staged with two segment counts and general, with a
    one-to-one map in between (the flag and the inverse map are cleared)."""
    x = W.gen_xfam(3, 2, 70000, 70000, 60000, dtype, seed=27)
    vm = x.vmap.copy()
    paired = np.flatnonzero(vm >= 0)
    rep = paired[1::5]
    vm[rep] = vm[paired[0::5][:len(rep)]]
    for general, segs in ((False, 0), (False, 4), (True, 0)):
        with _with_xfam(vwl, general, segs):
            check(vwl, x, vmap=vm, label="repeated ids general=%s segs=%d" % (general, segs))
            check(vwl, x, label="one-to-one general=%s segs=%d" % (general, segs))


