"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function ``include/vwl.h`` declares, sizes workspaces from the shape
alone, and its argument checks return the documented status codes."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vwl.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:vwl_status|size_t|int|char|void)\s*\**\s*(\w+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import vocab_wide_logit_amd as vwl
    return vwl.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("asym_verify", "rapid_verify", "vwl_asym_workspace_bytes",
              "vwl_rapid_workspace_bytes", "vwl_status_string", "vwl_workspace_reset"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import vocab_wide_logit_amd as vwl
    out = subprocess.run(["nm", "-D", "--defined-only", vwl.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in _declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(vwl.SYMBOLS) <= exported


def test_bench_helper_exports_its_declarations():
    """libvwl_bench.so (the streaming reference the benchmark compares
    against) exports what include/vwl_bench.h declares."""
    import vocab_wide_logit_amd as vwl
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "vwl_bench.h")).read(), flags=re.S)
    names = re.findall(r"^\s*int\s+(\w+)\s*\(", src, flags=re.M)
    assert names == ["vwl_bench_stream_read"]
    path = os.path.join(os.path.dirname(vwl.LIB_PATH), "libvwl_bench.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    blib = ctypes.CDLL(path)
    f = blib.vwl_bench_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    assert f(None, 16, None, 1, 64, 4, None) == 1          # null pointers, before any launch
    assert f(16, 16, 16, 1, 96, 4, None) == 2              # block not a multiple of 64
    assert f(16, 16, 16, 1, 64, 5, None) == 2              # unsupported unroll


def test_status_strings(lib):
    for code in range(9):
        s = lib.vwl_status_string(code).decode()
        assert s.startswith("VWL_")
    assert lib.vwl_version() >= 100


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    """asym_verify_noalloc checks the shape's workspace against its 16 MiB
    scratch before it touches any pointer or the device."""
    lib.asym_verify_noalloc.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 + [ctypes.c_float] * 2 + \
        [ctypes.c_void_p] * 8
    lib.asym_verify_noalloc.restype = ctypes.c_int
    need = lib.vwl_asym_workspace_bytes(2782, 0, 151936, 1)
    assert need > 16 << 20
    assert lib.asym_verify_noalloc(None, None, None, None, 2782, 0, 151936, 1, 1.0, 0.5,
                                   None, None, None, None, None, None, None, None) == 8
    assert lib.vwl_asym_workspace_bytes(256, 4, 151936, 1) <= 16 << 20


def test_workspace_sizes(lib):
    for (B, K, V, dt) in [(1, 0, 1, 0), (4, 2, 1024, 0), (64, 2, 151936, 1), (256, 4, 151936, 1)]:
        n = lib.vwl_asym_workspace_bytes(B, K, V, dt)
        assert n > 0 and n % 256 == 0
        # grows with rows
        assert lib.vwl_asym_workspace_bytes(B + 1, K, V, dt) >= n
    assert lib.vwl_rapid_workspace_bytes(16, 10, 128256, 0) > 0
    assert lib.vwl_asym_workspace_bytes(0, 2, 10, 0) == 0
    assert lib.vwl_asym_workspace_bytes(1, 64, 10, 0) == 0
    assert lib.vwl_asym_workspace_bytes(1, 2, 0, 0) == 0
    assert lib.vwl_asym_workspace_bytes(1, 2, 10, 7) == 0
    assert lib.vwl_rapid_workspace_bytes(1, -1, 10, 0) == 0


def test_lmhead_workspace_sizes(lib):
    """The LM-head path's two workspace sizes: the full one holds the fp32
    (a, b) pairs of whole 64-row and 128-token tiles beyond the minimal one
    (records and partials); both 256-byte multiples, 0 for invalid shapes."""
    for (B, K, V, Hd, Ht) in [(1, 0, 1, 64, 64), (3, 2, 1000, 128, 128), (64, 2, 151936, 2560, 5120)]:
        full = lib.vwl_asym_lmhead_workspace_bytes(B, K, V, Hd, Ht)
        small = lib.vwl_asym_lmhead_workspace_min_bytes(B, K, V, Hd, Ht)
        assert 0 < small < full and small % 256 == 0 and full % 256 == 0
        rows = -(-B * (K + 1) // 64) * 64
        assert full - small >= rows * (-(-V // 128) * 128) * 8
    for bad in [(0, 2, 10, 64, 64), (1, 2, 10, 96, 64), (1, 2, 10, 64, 32), (1, 64, 10, 64, 64)]:
        assert lib.vwl_asym_lmhead_workspace_bytes(*bad) == 0
        assert lib.vwl_asym_lmhead_workspace_min_bytes(*bad) == 0


def _p(addr):
    return ctypes.c_void_p(addr)


A = 0x10000  # 16-byte aligned fake device addresses (never dereferenced)


def _asym_check(lib, **kw):
    args = dict(a=A, b=A + 0x1000, t=A + 0x2000, draft=A + 0x3000, B=2, K=2, V=100, dt=0,
                beta=1.0, gamma=0.5, D=A + 0x4000, ge=A + 0x5000, acc=A + 0x6000, fused=A + 0x7000,
                alen=A + 0x8000, tok=A + 0x9000, ws=0x100000, wsb=4096, need=4096)
    args.update(kw)
    return lib.vwl_asym_check(_p(args["a"]), _p(args["b"]), _p(args["t"]), _p(args["draft"]),
                              args["B"], args["K"], args["V"], args["dt"], args["beta"], args["gamma"],
                              _p(args["D"]), _p(args["ge"]), _p(args["acc"]), _p(args["fused"]),
                              _p(args["alen"]), _p(args["tok"]), _p(args["ws"]), args["wsb"], args["need"])


def test_asym_check_codes(lib):
    assert _asym_check(lib) == 0
    assert _asym_check(lib, a=0) == 1
    assert _asym_check(lib, D=0) == 1
    assert _asym_check(lib, draft=0) == 1
    assert _asym_check(lib, draft=0, acc=0, K=0) == 0        # no drafts: both may be null
    assert _asym_check(lib, B=0) == 2
    assert _asym_check(lib, K=-1) == 2
    assert _asym_check(lib, K=64) == 2
    assert _asym_check(lib, V=0) == 2
    assert _asym_check(lib, dt=2) == 3
    assert _asym_check(lib, beta=float("nan")) == 4
    assert _asym_check(lib, beta=float("inf")) == 4
    assert _asym_check(lib, gamma=-0.1) == 4
    assert _asym_check(lib, gamma=float("inf")) == 4
    assert _asym_check(lib, beta=-3.0, gamma=0.0) == 0
    assert _asym_check(lib, a=A + 8) == 7
    assert _asym_check(lib, fused=A + 0x7002) == 7
    assert _asym_check(lib, ws=0x100010) == 7
    assert _asym_check(lib, wsb=100, need=4096) == 5
    assert _asym_check(lib, ws=0) == 5


def _rapid_check(lib, **kw):
    args = dict(z=A, y=A + 0x1000, draft=A + 0x3000, ua=A + 0x4000, us=A + 0x5000, B=2, G=3, V=100,
                dt=0, eta=5.0, T=1.0, acc=A + 0x6000, alen=A + 0x8000, tok=A + 0x9000,
                ws=0x100000, wsb=4096, need=4096)
    args.update(kw)
    return lib.vwl_rapid_check(_p(args["z"]), _p(args["y"]), _p(args["draft"]), _p(args["ua"]),
                               _p(args["us"]), args["B"], args["G"], args["V"], args["dt"], args["eta"],
                               args["T"], _p(args["acc"]), _p(args["alen"]), _p(args["tok"]),
                               _p(args["ws"]), args["wsb"], args["need"])


def test_rapid_check_codes(lib):
    assert _rapid_check(lib) == 0
    assert _rapid_check(lib, us=0) == 1
    assert _rapid_check(lib, ua=0) == 1
    assert _rapid_check(lib, ua=0, draft=0, acc=0, G=0) == 0
    assert _rapid_check(lib, G=64) == 2
    assert _rapid_check(lib, dt=9) == 3
    assert _rapid_check(lib, eta=-1.0) == 4
    assert _rapid_check(lib, T=0.0) == 4
    assert _rapid_check(lib, T=float("nan")) == 4
    assert _rapid_check(lib, z=A + 4) == 7
    assert _rapid_check(lib, us=A + 0x5002) == 7
    assert _rapid_check(lib, wsb=10) == 5


def test_plan_override_validation(lib):
    assert lib.vwl_set_plan_override(0, 3, 0) == 4
    assert lib.vwl_set_plan_override(2, 0, 0) == 4
    assert lib.vwl_set_plan_override(0, 0, -1) == 4
    assert lib.vwl_set_plan_override(0, 0, 0) == 0


def test_xfam_override_validation(lib):
    assert lib.vwl_set_xfam_override(2, 0) == 4
    assert lib.vwl_set_xfam_override(0, -1) == 4
    assert lib.vwl_set_xfam_override(0, 17) == 4
    assert lib.vwl_set_xfam_override(1, 16) == 0
    assert lib.vwl_set_xfam_override(0, 0) == 0


def test_bf16_marshalling_is_exact():
    """The binding's host->device bf16 conversion keeps the stored bits."""
    import torch
    x = W.round_to_bf16(np.random.default_rng(0).normal(0, 3, 4096).astype(np.float32))
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(t.view(torch.int16).numpy().view(np.uint16), W.bf16_bits(x))


def test_generator_structure():
    """Exact counts of the planted structure and drafts = argmax a."""
    x = W.gen_asym(20, 4, 700, "bf16", seed=3, displaced_frac=0.3, identical_frac=0.2, tie_frac=0.05)
    R = 100
    assert x.identical.sum() == round(0.2 * R)
    assert x.tie.sum() == round(0.05 * R)
    assert x.displaced.sum() == round(0.3 * R)
    assert not np.any(x.identical & x.tie)
    assert np.array_equal(x.b[x.identical], x.a[x.identical])
    np.testing.assert_array_equal(x.draft, np.argmax(x.a[:, :4], axis=2))
    W.bf16_bits(x.a)  # bf16-exact
    r = W.gen_rapid(3, 4, 500, seed=9)
    assert r.displaced.sum() == round(0.4 * 15)
    assert r.u_accept.dtype == np.float32 and np.all(r.u_accept < 1.0)
    assert np.all((r.u_sample * 2 ** 24) == np.round(r.u_sample * 2 ** 24))
    # same seed, same data; generation does not depend on the thread count
    x2 = W.gen_asym(20, 4, 700, "bf16", seed=3, displaced_frac=0.3, identical_frac=0.2, tie_frac=0.05)
    assert np.array_equal(x.a, x2.a) and np.array_equal(x.t, x2.t)


def test_phase_event_hook_accepts_null(lib):
    assert lib.vwl_set_phase_event(None) == 0


def test_rapid_vocabulary_limit(lib):
    """RAPID rejects V above VWL_RAPID_MAX_V (the tail's geometry limit)."""
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vwl.h")).read()
    vmax = int(re.search(r"#define VWL_RAPID_MAX_V (\d+)", hdr).group(1))
    assert lib.vwl_rapid_workspace_bytes(1, 1, vmax, 0) > 0
    p = ctypes.c_void_p(256)
    args = lambda V: (p, p, p, p, p, 1, 1, V, 0, ctypes.c_float(1.0), ctypes.c_float(1.0), p, p, p, p,
                      ctypes.c_size_t(1 << 40), ctypes.c_size_t(1))
    assert lib.vwl_rapid_check(*args(vmax)) == 0
    assert lib.vwl_rapid_check(*args(vmax + 1)) == 2


def _variant(lib, a, delta, gate, ws):
    """asym_verify_variant with placeholder device pointers: every case here
    returns from the host-side checks, before anything touches a device."""
    p = lambda x: ctypes.c_void_p(x) if x else None
    return lib.asym_verify_variant(p(a), p(A + 0x1000), p(A + 0x2000), p(A + 0x3000), 2, 2, 100, 0,
                                   ctypes.c_float(1.0), ctypes.c_float(0.5), delta, gate,
                                   p(A + 0x4000), p(A + 0x5000), p(A + 0x6000), p(A + 0x7000),
                                   p(A + 0x8000), p(A + 0x9000), None, p(ws), ctypes.c_size_t(0), None)


def test_asym_variant_argument_codes(lib):
    """Unknown fusion source or gate: VWL_ERR_PARAM; a is required except
    for the fixed gate with delta = t - b (which then fails only on the
    missing workspace)."""
    assert _variant(lib, A, 3, 0, 0) == 4
    assert _variant(lib, A, -1, 0, 0) == 4
    assert _variant(lib, A, 0, 2, 0) == 4
    for delta in (0, 1, 2):
        assert _variant(lib, 0, delta, 0, 0) == 1
    assert _variant(lib, 0, 0, 1, 0) == 1
    assert _variant(lib, 0, 1, 1, 0) == 1
    assert _variant(lib, 0, 2, 1, 0) == 5
    assert _variant(lib, A, 2, 1, 0) == 5


def _e2sci(lib, **kw):
    """e2sci_verify with placeholder device pointers: every case here returns
    from the host-side checks, before anything touches a device."""
    args = dict(y=A, z=A + 0x1000, B=2, W=4, V=100, dt=0, T=A + 0x2000, om=A + 0x3000, r=A + 0x4000,
                age=0, prm=(1.0, 0.5, 0.1, 0.01, 0.3, 0.3), D=A + 0x5000, acc=A + 0x6000, alen=A + 0x7000,
                To=A + 0x8000, ws=0, wsb=0)
    args.update(kw)
    p = lambda x: ctypes.c_void_p(x) if x else None
    import vocab_wide_logit_amd as vwl
    prm = None if args["prm"] is None else ctypes.byref(vwl.E2sciParams(*args["prm"]))
    return lib.e2sci_verify(p(args["y"]), p(args["z"]), args["B"], args["W"], args["V"], args["dt"],
                            p(args["T"]), p(args["om"]), p(args["r"]), p(args["age"]), prm, p(args["D"]),
                            p(args["acc"]),
                            p(args["alen"]), p(args["To"]), None, p(args["ws"]), ctypes.c_size_t(args["wsb"]),
                            None)


def test_e2sci_argument_codes(lib):
    assert lib.vwl_e2sci_workspace_bytes(2, 4, 100, 0) > 0
    assert lib.vwl_e2sci_workspace_bytes(2, 0, 100, 0) == 0
    assert _e2sci(lib) == 5                      # all good but no workspace
    for k in ("y", "z", "T", "om", "r", "D", "acc", "alen", "To"):
        assert _e2sci(lib, **{k: 0}) == 1, k
    assert _e2sci(lib, prm=None) == 1
    assert _e2sci(lib, W=0) == 2
    assert _e2sci(lib, W=65) == 2
    assert _e2sci(lib, B=0) == 2
    assert _e2sci(lib, dt=5) == 3
    assert _e2sci(lib, prm=(1.0, 0.5, 0.1, 0.3, 0.01, 0.3)) == 4      # T_min > T_max
    assert _e2sci(lib, prm=(1.0, 0.5, 0.1, 0.01, 0.3, 1.5)) == 4      # ewma outside [0, 1]
    assert _e2sci(lib, prm=(float("nan"), 0.5, 0.1, 0.01, 0.3, 0.3)) == 4
    assert _e2sci(lib, y=A + 4) == 7
    assert _e2sci(lib, T=A + 0x2002) == 7
    # the stabilisers: hysteresis >= 0, min_refresh >= 0, T_safe within [T_min, T_max] when delta > 0,
    # a count array when min_refresh > 1
    base = (1.0, 0.5, 0.1, 0.01, 0.3, 0.3)
    assert _e2sci(lib, prm=base + (0.01, 1, 0.25, 0.05)) == 5
    assert _e2sci(lib, prm=base + (-0.01, 1, 0.0, 0.0)) == 4
    assert _e2sci(lib, prm=base + (float("inf"), 1, 0.0, 0.0)) == 4
    assert _e2sci(lib, prm=base + (0.0, -1, 0.0, 0.0)) == 4
    assert _e2sci(lib, prm=base + (0.0, 1, 0.25, 0.5)) == 4
    assert _e2sci(lib, prm=base + (0.0, 1, 0.25, 0.001)) == 4
    assert _e2sci(lib, prm=base + (0.0, 1, 0.0, 0.5)) == 5            # delta 0: T_safe unused
    assert _e2sci(lib, prm=base + (0.0, 1, float("nan"), 0.05)) == 4
    assert _e2sci(lib, prm=base + (0.0, 3, 0.0, 0.0)) == 1            # min_refresh 3 needs age
    assert _e2sci(lib, prm=base + (0.0, 3, 0.0, 0.0), age=A + 0x9000) == 5
    assert _e2sci(lib, prm=base + (0.0, 3, 0.0, 0.0), age=A + 0x9002) == 7


def test_asym_xfam_argument_codes(lib):
    """Host-side checks of the cross-family entry point (no device access)."""
    p = lambda x: ctypes.c_void_p(x) if x else None

    def call(a=A, vmap=A + 0xA000, Vd=100, Vt=90, B=2, K=2, dt=0, ws=0, wsb=0):
        return lib.asym_verify_xfam(p(a), p(A + 0x1000), Vd, p(A + 0x2000), Vt, p(vmap), p(A + 0x3000), B, K, dt,
                                    ctypes.c_float(1.0), ctypes.c_float(0.5), p(A + 0x4000), p(A + 0x5000),
                                    p(A + 0x6000), p(A + 0x7000), p(A + 0x8000), p(A + 0x9000), None, p(ws),
                                    ctypes.c_size_t(wsb), None)

    assert lib.vwl_asym_xfam_workspace_bytes(2, 2, 100, 90, 0) > lib.vwl_asym_workspace_bytes(2, 2, 100, 0)
    assert lib.vwl_asym_xfam_workspace_bytes(2, 2, 100, 0, 0) == 0
    assert call() == 5          # everything valid except the missing workspace
    assert call(vmap=0) == 1
    assert call(a=0) == 1
    assert call(Vt=0) == 2
    assert call(Vd=0) == 2
    assert call(dt=4) == 3
    assert call(vmap=A + 0xA002, ws=0x100000, wsb=1 << 30) == 7


def test_divergence_polynomial_constants():
    """The one-exponential divergence term of the kernels: the fp32 Horner
    evaluation of u * P(u) with the coefficients compiled into the HIP
    source matches Psi(x)/2 = cosh(x/2) (x tanh(x/2) - 2 ln cosh(x/2)) / 2
    (evaluated in fp64) within 4e-7 relative on |x| < kPsiX1, the range the
    kernels use it on; the identity itself, for one element with x = ln p -
    ln q, gives that element's share of the JSD, checked here on random
    (p, q)."""
    import re
    src = open(os.path.join(ROOT, "vocab_wide_logit_amd", "csrc", "asym_kernels.hpp")).read()
    x1 = float(re.search(r"constexpr float kPsiX1 = ([0-9.]+)f;", src).group(1))
    cf = {int(k): float.fromhex(v) for k, v in re.findall(r"constexpr float kPsiP(\d) = (-?0x[0-9a-fA-Fp.+-]+)f;", src)}
    deg = max(cf)
    assert sorted(cf) == list(range(deg + 1))
    x = np.linspace(1e-3, x1 * (1 - 1e-7), 200001)
    u = (((x.astype(np.float32) * np.float32(1.0 / x1))) ** 2).astype(np.float32)
    acc = np.float32(cf[deg])
    for k in range(deg - 1, -1, -1):
        acc = (acc * u + np.float32(cf[k])).astype(np.float32)
    val = (acc * u).astype(np.float64)
    xu = x1 * np.sqrt(u.astype(np.float64))
    exact = np.cosh(xu / 2) * (xu * np.tanh(xu / 2) - 2 * np.log(np.cosh(xu / 2))) / 2
    assert np.max(np.abs(val / exact - 1)) < 4e-7
    rng = np.random.default_rng(5)
    p, q = rng.uniform(1e-6, 1, 1000), rng.uniform(1e-6, 1, 1000)
    xs = np.log(p) - np.log(q)
    share = (p * np.log(2 * p / (p + q)) + q * np.log(2 * q / (p + q))) / 2
    psi = np.cosh(xs / 2) * (xs * np.tanh(xs / 2) - 2 * np.log(np.cosh(xs / 2)))
    np.testing.assert_allclose(np.sqrt(p * q) * psi / 2, share, rtol=1e-9, atol=1e-15)


def test_binding_drops_cached_workspaces_after_a_timeout():
    """The binding's workspace cache: drop_workspaces() empties it, and
    check_dev_err() drops it exactly when the timeout bit is set (host-side
    logic only; the tensors here live on the CPU)."""
    import torch
    import vocab_wide_logit_amd as vwl
    vwl.drop_workspaces()
    vwl._ws_cache[("probe", 1)] = torch.zeros(4, dtype=torch.uint8)
    assert vwl.check_dev_err(torch.tensor([vwl.VWL_DEVERR_DRAFT | vwl.VWL_DEVERR_UNIFORM], dtype=torch.int32)) == 3
    assert len(vwl._ws_cache) == 1
    assert vwl.check_dev_err(torch.tensor([vwl.VWL_DEVERR_TIMEOUT], dtype=torch.int32)) == 4
    assert len(vwl._ws_cache) == 0
    vwl._ws_cache[("probe", 2)] = torch.zeros(4, dtype=torch.uint8)
    assert vwl.drop_workspaces() == 1 and not vwl._ws_cache
