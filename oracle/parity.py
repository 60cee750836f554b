"""Comparison rules between the device outputs and the fp64 oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark report).

Rules:
* AsymSpec acceptance flags, accept lengths and emitted tokens are compared
  bit for bit.  A draft whose log-space margin
  ``log p_t(d) - log p_b(d) - log gamma + D`` is within 1e-6 of zero is
  "margin-ambiguous"; a fused token whose fp64 score gap to the runner-up is
  in (0, 1e-6 * max(|top1|, 1)] is "gap-ambiguous" (exact ties are never
  ambiguous: the lowest index must win).  A request is excluded, and counted,
  when a decisive position (i <= accept length) or its emitted token is
  ambiguous.
* D and gamma_eff: within 1e-5 relative plus an absolute floor of 1e-9 for
  D (a relative bound is void at D = 0, which a single-token row or two rows
  that differ by a constant reach exactly in the oracle); for drafter rows
  that are bitwise identical the device must return exactly 0 and gamma.
* E2-SCI: D as above; a position is ambiguous when its divergence is within
  1e-5 relative of the window threshold; the credit state and the next
  threshold within 1e-6 relative on the requests whose decisive positions
  are clear.
* RAPID: a draft test is ambiguous when |u*q - phat| <= 1e-6 * max(u*q, phat)
  or the draft's augmented logit is within 1e-6 of the tail threshold; a draw
  is ambiguous when u*S is within 1e-6*S of an end of the chosen interval or
  a token of the emitting row sits within 1e-6 of the tail threshold.
  phat and q at the drafts: 1e-5 relative.  The emitted distribution:
  |dev - ora| <= 1e-5 * ora + 4 * 2^-24 * (p + max(phat, q)) / S elementwise.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

MARGIN_EPS = 1e-6
GAP_EPS = 1e-6
REL_TOL = 1e-5
D_ABS_FLOOR = 1e-9
RAPID_EPS = 1e-6


@dataclass
class Report:
    ok: bool = True
    checked: int = 0
    excluded: int = 0
    problems: list = field(default_factory=list)
    stats: dict = field(default_factory=dict)

    def fail(self, msg: str):
        self.ok = False
        if len(self.problems) < 20:
            self.problems.append(msg)

    def __str__(self):
        return "ok=%s checked=%d excluded=%d stats=%s problems=%s" % (
            self.ok, self.checked, self.excluded, self.stats, self.problems[:5])


def _rel_close(dev, ref, rtol):
    dev = np.asarray(dev, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(dev - ref) <= rtol * np.abs(ref) + 1e-300


def compare_asym(dev: dict, ora, K: int, rtol: float = REL_TOL, identical=None,
                 d_floor: float = D_ABS_FLOOR, gate: str = "cda") -> Report:
    """dev: numpy arrays D, gamma_eff, accept, fused, accept_len, token;
    ora: oracle.AsymResult; identical: bool [B, K+1], rows whose two drafter
    views are bitwise equal.  Under the fixed gate the device reports no D
    (NaN) and gamma_eff must be gamma exactly."""
    rep = Report()
    D_o, D_d = ora.D, np.asarray(dev["D"], np.float64)
    g_o = ora.gamma_eff
    g_d = np.asarray(dev["gamma_eff"], np.float64)
    if gate == "fixed":
        if not np.all(np.isnan(D_d)):
            rep.fail("D must be NaN under the fixed gate")
        if np.any(g_d != g_o):
            rep.fail("gamma_eff must be gamma exactly under the fixed gate")
        return _compare_asym_decisions(rep, dev, ora, K)
    if identical is not None:
        ident = np.asarray(identical, bool)
        if np.any(D_d[ident] != 0.0):
            rep.fail("D must be exactly 0 for identical drafter rows (%d rows)" % int(np.sum(D_d[ident] != 0.0)))
        if np.any(g_d[ident] != np.float32(g_o[ident]).astype(np.float64)):
            rep.fail("gamma_eff must equal gamma exactly for identical drafter rows")
    zero = D_o == 0.0
    nz = ~zero
    badz = np.abs(D_d[zero]) > d_floor
    if np.any(badz):
        rep.fail("|D| above %g where the oracle's D is 0 (%d rows)" % (d_floor, int(badz.sum())))
    bad = np.abs(D_d[nz] - D_o[nz]) > rtol * np.abs(D_o[nz]) + d_floor
    if np.any(bad):
        rep.fail("D outside %g relative on %d rows (max rel %.3g)" % (
            rtol, int(bad.sum()), float(np.max(np.abs(D_d[nz] - D_o[nz]) / np.abs(D_o[nz])))))
    badg = ~_rel_close(g_d, g_o, rtol)
    if np.any(badg):
        rep.fail("gamma_eff outside %g relative on %d rows" % (rtol, int(badg.sum())))
    rep.stats["D_max_rel"] = float(np.max(np.abs(D_d[nz] - D_o[nz]) / np.abs(D_o[nz]))) if np.any(nz) else 0.0
    return _compare_asym_decisions(rep, dev, ora, K)


def _compare_asym_decisions(rep: Report, dev: dict, ora, K: int) -> Report:
    """Fused tokens, acceptance flags, accept lengths and emitted tokens."""
    # fused tokens
    gap = ora.gap
    top = np.maximum(np.abs(ora.top), 1.0)
    amb_f = (gap > 0.0) & (gap <= GAP_EPS * top)
    f_d = np.asarray(dev["fused"])
    mism_f = (f_d != ora.fused) & ~amb_f
    if np.any(mism_f):
        rep.fail("fused token mismatch on %d rows (first %s)" % (int(mism_f.sum()), np.argwhere(mism_f)[0].tolist()))
    rep.stats["fused_ambiguous"] = int(amb_f.sum())
    rep.stats["exact_ties"] = int((gap == 0.0).sum())

    # acceptance and scan
    B = f_d.shape[0]
    if K > 0:
        amb_a = np.abs(ora.margin) <= MARGIN_EPS
        a_d = np.asarray(dev["accept"]).astype(np.uint8)
        mism_a = (a_d != ora.accept) & ~amb_a
        if np.any(mism_a):
            rep.fail("accept mismatch on %d drafts (first %s)" % (int(mism_a.sum()), np.argwhere(mism_a)[0].tolist()))
        rep.stats["accept_ambiguous"] = int(amb_a.sum())
        rep.stats["acceptance_rate"] = float(ora.accept.mean())
    else:
        amb_a = np.zeros((B, 0), bool)
    al_d = np.asarray(dev["accept_len"])
    tok_d = np.asarray(dev["token"])
    for bi in range(B):
        n = int(ora.accept_len[bi])
        decisive = amb_a[bi, :min(n + 1, K)].any() if K > 0 else False
        if decisive or amb_f[bi, n]:
            rep.excluded += 1
            continue
        rep.checked += 1
        if al_d[bi] != n:
            rep.fail("accept_len mismatch at request %d: dev %d oracle %d" % (bi, al_d[bi], n))
        if tok_d[bi] != ora.token[bi]:
            rep.fail("token mismatch at request %d: dev %d oracle %d" % (bi, tok_d[bi], ora.token[bi]))
    rep.stats["mean_accept_len"] = float(ora.accept_len.mean())
    return rep


def compare_rapid(dev: dict, ora, G: int, u_accept=None, rtol: float = REL_TOL) -> Report:
    """dev: numpy arrays accept, accept_len, token and optionally p_hat_draft,
    q_draft, emit_dist; ora: oracle.RapidResult (emit_dist needed for the
    distribution check)."""
    rep = Report()
    B = ora.accept_len.shape[0]
    if G > 0:
        amb_a = (ora.acc_rel <= RAPID_EPS) | (ora.tail_d_dist <= RAPID_EPS)
        a_d = np.asarray(dev["accept"]).astype(np.uint8)
        mism = (a_d != ora.accept) & ~amb_a
        if np.any(mism):
            rep.fail("accept mismatch on %d drafts (first %s)" % (int(mism.sum()), np.argwhere(mism)[0].tolist()))
        rep.stats["accept_ambiguous"] = int(amb_a.sum())
        rep.stats["acceptance_rate"] = float(ora.accept.mean())
        valid = np.isfinite(ora.tail_d_dist) & (ora.tail_d_dist > RAPID_EPS)
        for key, ref in (("p_hat_draft", ora.phat_draft), ("q_draft", ora.q_draft)):
            if dev.get(key) is not None:
                d = np.asarray(dev[key], np.float64)
                bad = valid & ~_rel_close(d, ref, rtol)
                if np.any(bad):
                    rep.fail("%s outside %g relative on %d drafts" % (key, rtol, int(bad.sum())))
                if np.any(valid):
                    rep.stats[key + "_max_rel"] = float(np.max(np.abs(d[valid] - ref[valid]) / np.abs(ref[valid])))
    else:
        amb_a = np.zeros((B, 0), bool)
    al_d = np.asarray(dev["accept_len"])
    tok_d = np.asarray(dev["token"])
    tight = 0
    for bi in range(B):
        n = int(ora.accept_len[bi])
        if G > 0 and amb_a[bi, :min(n + 1, G)].any():
            rep.excluded += 1
            continue
        if al_d[bi] != n:
            rep.fail("accept_len mismatch at request %d: dev %d oracle %d" % (bi, al_d[bi], n))
            continue
        if ora.draw_slack[bi] <= RAPID_EPS or ora.tail_close[bi] > 0:
            rep.excluded += 1
            if tok_d[bi] == ora.token[bi]:
                tight += 1
            continue
        rep.checked += 1
        if tok_d[bi] != ora.token[bi]:
            rep.fail("token mismatch at request %d: dev %d oracle %d (slack %.3g)" % (
                bi, tok_d[bi], ora.token[bi], ora.draw_slack[bi]))
    rep.stats["excluded_draws_still_equal"] = tight
    if dev.get("emit_dist") is not None and ora.emit_dist is not None:
        d = np.asarray(dev["emit_dist"], np.float64)
        o = ora.emit_dist
        S = np.where(ora.resid_S > 0, ora.resid_S, 1.0)[:, None]
        allow = rtol * o + 4 * 2.0 ** -24 * ora.emit_scale / S
        ok_rows = np.ones(B, bool)
        for bi in range(B):
            n = int(ora.accept_len[bi])
            if (G > 0 and amb_a[bi, :min(n + 1, G)].any()) or ora.tail_close[bi] > 0:
                ok_rows[bi] = False
        bad = (np.abs(d - o) > allow) & ok_rows[:, None]
        if np.any(bad):
            rep.fail("emit_dist outside tolerance on %d entries" % int(bad.sum()))
        rep.stats["emit_tv_max"] = float(np.max(0.5 * np.sum(np.abs(d - o), axis=1)[ok_rows])) if ok_rows.any() else 0.0
        rep.stats["emit_rel_max"] = float(np.max((np.abs(d - o) / np.maximum(o, 1e-30))[ok_rows][o[ok_rows] > 1e-7])) if ok_rows.any() else 0.0
    return rep


def compare_e2sci(dev: dict, ora, T, identical=None, rtol: float = REL_TOL,
                  d_floor: float = D_ABS_FLOOR, state_rtol: float = 1e-6) -> Report:
    """dev: numpy arrays D, accept, accept_len, T_next, r_hat; ora:
    oracle.E2sciResult; T: [B] thresholds of the window.  A position whose
    oracle divergence is within 1e-5 relative (plus 1e-9) of its threshold is
    ambiguous; a request is excluded, and counted, when a decisive position
    (i <= accept length) is.  The credit state and the next threshold are
    compared within 1e-6 relative (plus 1e-7) on the requests checked.  With
    the stabilisers on, a request whose dead-band decision lies within 1e-9 of
    the band (|T_prop - T_in| - hysteresis) is excluded too, and the device's
    window count, when given (dev["age"]), must equal the oracle's."""
    rep = Report()
    D_o, D_d = ora.D, np.asarray(dev["D"], np.float64)
    if identical is not None:
        ident = np.asarray(identical, bool)
        if np.any(D_d[ident] != 0.0):
            rep.fail("D must be exactly 0 for identical rows (%d rows)" % int(np.sum(D_d[ident] != 0.0)))
    zero = D_o == 0.0
    if np.any(np.abs(D_d[zero]) > d_floor):
        rep.fail("|D| above %g where the oracle's D is 0" % d_floor)
    nz = ~zero
    bad = np.abs(D_d[nz] - D_o[nz]) > rtol * np.abs(D_o[nz]) + d_floor
    if np.any(bad):
        rep.fail("D outside %g relative on %d rows" % (rtol, int(bad.sum())))
    rep.stats["D_max_rel"] = float(np.max(np.abs(D_d[nz] - D_o[nz]) / np.abs(D_o[nz]))) if np.any(nz) else 0.0
    T = np.asarray(T, np.float64).reshape(-1, 1)
    amb = np.abs(D_o - T) <= rtol * np.maximum(np.abs(D_o), np.abs(T)) + d_floor
    a_d = np.asarray(dev["accept"]).astype(np.uint8)
    mism = (a_d != ora.accept) & ~amb
    if np.any(mism):
        rep.fail("accept mismatch on %d positions (first %s)" % (int(mism.sum()), np.argwhere(mism)[0].tolist()))
    rep.stats["accept_ambiguous"] = int(amb.sum())
    rep.stats["acceptance_rate"] = float(ora.accept.mean())
    al_d = np.asarray(dev["accept_len"])
    r_d = np.asarray(dev["r_hat"], np.float64)
    t_d = np.asarray(dev["T_next"], np.float64)
    age_d = dev.get("age")
    hm = getattr(ora, "hyst_margin", None)
    Wn = D_o.shape[1]
    for bi in range(D_o.shape[0]):
        n = int(ora.accept_len[bi])
        if amb[bi, :min(n + 1, Wn)].any() or (hm is not None and abs(hm[bi]) <= 1e-9):
            rep.excluded += 1
            continue
        if age_d is not None and int(age_d[bi]) != int(ora.age[bi]):
            rep.fail("age mismatch at request %d: dev %d oracle %d" % (bi, int(age_d[bi]), int(ora.age[bi])))
        rep.checked += 1
        if al_d[bi] != n:
            rep.fail("accept_len mismatch at request %d: dev %d oracle %d" % (bi, al_d[bi], n))
        if abs(r_d[bi] - ora.r_hat[bi]) > state_rtol * abs(ora.r_hat[bi]) + 1e-7:
            rep.fail("r_hat mismatch at request %d: dev %r oracle %r" % (bi, r_d[bi], ora.r_hat[bi]))
        if abs(t_d[bi] - ora.T_next[bi]) > state_rtol * abs(ora.T_next[bi]) + 1e-7:
            rep.fail("T_next mismatch at request %d: dev %r oracle %r" % (bi, t_d[bi], ora.T_next[bi]))
    return rep


def compare_lmhead(dev: dict, lm, K: int, beta: float, rtol: float = REL_TOL) -> Report:
    """AsymSpec from hidden states: the device's logits carry the error of an
    fp32 product-sum, bounded per logit by the oracle (lm: oracle.LmheadResult,
    row maxima err_a, err_b, err_t).  The windows widen by those bounds: a
    logit error e moves a log-sum-exp by at most e, the JSD by at most
    2 (e_a + e_b), a margin (draft logits exact) by e_t + e_b + 2 (e_a + e_b),
    and a fused score by e_t + |beta| (e_a + e_b)."""
    ora = lm.res
    rep = Report()
    ea, eb, et = lm.err_a, lm.err_b, lm.err_t
    dD = 2.0 * (ea + eb)
    D_d = np.asarray(dev["D"], np.float64)
    bad = np.abs(D_d - ora.D) > rtol * np.abs(ora.D) + dD + D_ABS_FLOOR
    if np.any(bad):
        rep.fail("D outside its window on %d rows" % int(bad.sum()))
    g_d = np.asarray(dev["gamma_eff"], np.float64)
    badg = np.abs(g_d - ora.gamma_eff) > (rtol + dD) * np.abs(ora.gamma_eff) + 1e-30
    if np.any(badg):
        rep.fail("gamma_eff outside its window on %d rows" % int(badg.sum()))
    rep.stats["D_max_abs"] = float(np.max(np.abs(D_d - ora.D)))
    rep.stats["D_window_max"] = float(np.max(dD))
    gap_w = 2.0 * (et + abs(beta) * (ea + eb)) + GAP_EPS * np.maximum(np.abs(ora.top), 1.0)
    amb_f = (ora.gap > 0.0) & (ora.gap <= gap_w)
    f_d = np.asarray(dev["fused"])
    mism_f = (f_d != ora.fused) & ~amb_f
    if np.any(mism_f):
        rep.fail("fused token mismatch on %d rows (first %s)" % (int(mism_f.sum()), np.argwhere(mism_f)[0].tolist()))
    rep.stats["fused_ambiguous"] = int(amb_f.sum())
    B = f_d.shape[0]
    if K > 0:
        m_w = (et + eb + dD)[:, :K] + MARGIN_EPS
        amb_a = np.abs(ora.margin) <= m_w
        a_d = np.asarray(dev["accept"]).astype(np.uint8)
        mism_a = (a_d != ora.accept) & ~amb_a
        if np.any(mism_a):
            rep.fail("accept mismatch on %d drafts (first %s)" % (int(mism_a.sum()), np.argwhere(mism_a)[0].tolist()))
        rep.stats["accept_ambiguous"] = int(amb_a.sum())
        rep.stats["acceptance_rate"] = float(ora.accept.mean())
    else:
        amb_a = np.zeros((B, 0), bool)
    al_d = np.asarray(dev["accept_len"])
    tok_d = np.asarray(dev["token"])
    for bi in range(B):
        n = int(ora.accept_len[bi])
        if (K > 0 and amb_a[bi, :min(n + 1, K)].any()) or amb_f[bi, n]:
            rep.excluded += 1
            continue
        rep.checked += 1
        if al_d[bi] != n:
            rep.fail("accept_len mismatch at request %d: dev %d oracle %d" % (bi, al_d[bi], n))
        if tok_d[bi] != ora.token[bi]:
            rep.fail("token mismatch at request %d: dev %d oracle %d" % (bi, tok_d[bi], ora.token[bi]))
    return rep
