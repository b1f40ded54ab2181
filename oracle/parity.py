"""Comparison of the GPU library's outputs with the CPU oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check).  Receives plain arrays; never
imports or calls the GPU library.

Greedy and candidate results must be bit-exact.  Sampling results must match
exactly, except in rounds where the oracle's own decision lies within `eps`
of its boundary, where float32 rounding on the GPU may legitimately go the
other way:
  - an acceptance decision with |u_i - min(1, p/q)| < eps: the rounds may
    then diverge from that position on (the accepted drafts before it must
    still agree);
  - the round's draw with u_k within eps of a boundary of the drawn token's
    CDF interval: the GPU's token must then be a token of positive weight
    whose own interval lies within eps of u_k.
Such rounds are counted, not hidden.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import (draw_interval, greedy, greedy_candidates, greedy_matches, row_argmax, sample,
               sample_lenient, sample_truncated, token_probs, truncated_row)


@dataclasses.dataclass
class SampleReport:
    rounds: int = 0
    exact: int = 0
    tie_accept: int = 0
    tie_sample: int = 0
    tie_trunc: int = 0
    failures: list = dataclasses.field(default_factory=list)
    committed: int = 0

    def ok(self):
        return not self.failures

    def summary(self):
        return (f"rounds={self.rounds} exact={self.exact} tie_accept={self.tie_accept} "
                f"tie_sample={self.tie_sample} tie_trunc={self.tie_trunc} "
                f"failures={len(self.failures)} "
                f"mean_committed={self.committed / max(1, self.rounds):.4f}")


def check_sample(z, y, x, u, T, gpu_tokens, gpu_nacc, eps=1e-5, report=None,
                 seq_ids=None, lenience=None) -> SampleReport:
    """z [B,k+1,V], y [B,k,V] float32; x [B,k]; u [B,k+1]; GPU outputs as numpy.
    `lenience` (l >= 1) compares against the lenient rule instead."""
    rep = report or SampleReport()
    if lenience is None:
        ot, on, tr = sample(z, y, x, u, T, traces=True)
    else:
        ot, on, tr = sample_lenient(z, y, x, u, T, lenience, traces=True)
    B, k1 = ot.shape
    k = k1 - 1
    for b in range(B):
        sid = b if seq_ids is None else seq_ids[b]
        rep.rounds += 1
        rep.committed += int(gpu_nacc[b]) + 1
        gt, gn = gpu_tokens[b], int(gpu_nacc[b])
        if gn == on[b] and (gt == ot[b]).all():
            rep.exact += 1
            continue
        t = tr[b]
        first = min(gn, int(on[b]))
        if not (0 <= gn <= k) or not (gt[:first] == ot[b, :first]).all():
            rep.failures.append((sid, "accepted prefix differs", gt.tolist(), ot[b].tolist()))
            continue
        if (gt[gn + 1:] != -1).any():
            rep.failures.append((sid, "padding", gt.tolist(), ot[b].tolist()))
            continue
        if gn != on[b]:
            if first < t.evaluated and t.accept_margin[first] < eps:
                rep.tie_accept += 1
            else:
                rep.failures.append((sid, f"accepted length {gn} vs {on[b]}", gt.tolist(),
                                     ot[b].tolist(), t.accept_margin[first]))
            continue
        j = gn
        if t.sample_margin < eps:
            lo, hi, w = draw_interval(z[b, j], y[b, j] if j < k else None, T, int(gt[j])) \
                if 0 <= gt[j] < z.shape[2] else (0.0, 0.0, 0.0)
            if w > 0 and lo - eps <= u[b, k] <= hi + eps:
                rep.tie_sample += 1
                continue
        rep.failures.append((sid, f"drawn token {gt[j]} vs {ot[b, j]}", float(u[b, k]),
                             t.sample_lo, t.sample_hi, t.sample_margin))
    return rep


# The exported p(x), q(x) are float32: below float32's smallest normal number
# a value cannot carry relative precision (and underflows to 0 below 2^-149),
# so there the error is measured against that number instead of the value.
FP32_MIN_NORMAL = 2.0 ** -126


def prob_error(got, ref):
    """Relative error of float32 probabilities, with float32's smallest normal
    number as the floor of the denominator."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.abs(got - ref) / np.maximum(ref, FP32_MIN_NORMAL)


def check_probs(z, y, x, T, gpu_px, gpu_qx, rtol=1e-5):
    """Largest error of the exported p_i(x_i), q_i(x_i) over all positions
    (relative, and absolute below float32's normal range: prob_error).  A
    token the oracle gives probability 0 must be exported as exactly 0."""
    worst = 0.0
    for b in range(z.shape[0]):
        px, qx = token_probs(z[b], y[b], x[b], T)
        for ref, got in ((px, gpu_px[b]), (qx, gpu_qx[b])):
            zero = ref == 0
            if (got[zero] != 0).any():
                return float("inf")
            if (~zero).any():
                worst = max(worst, float(prob_error(got[~zero], ref[~zero]).max()))
    return worst


def check_greedy(z, x, gpu_tokens, gpu_nacc):
    """Bit-exact comparison; returns the list of mismatching sequence indices."""
    ot, on = greedy(z, x)
    bad = np.nonzero((on != gpu_nacc) | (ot != gpu_tokens).any(axis=1))[0]
    return bad.tolist(), ot, on


def check_candidates(z, cand, gpu_tokens, gpu_A, gpu_best):
    ot, oa, ob = greedy_candidates(z, cand)
    bad = np.nonzero((oa != gpu_A) | (ob != gpu_best) | (ot != gpu_tokens).any(axis=1))[0]
    return bad.tolist(), ot, oa, ob


def check_greedy_matches(z, x, gpu_v, gpu_mask, gpu_count):
    """Bit-exact comparison of the #Match by-products; returns mismatching rows."""
    v, mask, cnt = greedy_matches(z, x)
    gm = np.asarray(gpu_mask).astype(np.int64).view(np.uint64)
    bad = np.nonzero((v != gpu_v).any(axis=1) | (mask != gm) | (cnt != gpu_count))[0]
    return bad.tolist()


def check_row_argmax(z, gpu_v):
    ref = row_argmax(z)
    return np.argwhere(ref != gpu_v).tolist()


def _truncated_interval(zrow, yrow, T, top_k, top_p, token):
    """(lo, hi, weight) of `token` in the cumulative distribution drawn from on
    truncated rows: max(0, p' - q') against `yrow`, or p' if yrow is None."""
    p, _ = truncated_row(zrow, T, top_k, top_p)
    w = p
    if yrow is not None:
        q, _ = truncated_row(yrow, T, top_k, top_p)
        w = np.maximum(p - q, 0.0)
        if not w.sum() > 0:
            w = p
    cum = np.cumsum(w)
    S = cum[-1]
    lo = (cum[token] - w[token]) / S
    return lo, cum[token] / S, w[token]


def check_sample_truncated(z, y, x, u, T, top_k, top_p, gpu_tokens, gpu_nacc, eps=1e-5,
                           eps_trunc=1e-5, report=None) -> SampleReport:
    """As check_sample, on top-k / top-p truncated rows.  A round in which some
    row's top-p boundary lies within eps_trunc of top_p (the oracle's
    trunc_margin) may keep a different set on the GPU: it is counted as
    tie_trunc and checked for validity only (accepted drafts, padding)."""
    rep = report or SampleReport()
    ot, on, tr, margin = sample_truncated(z, y, x, u, T, top_k, top_p, traces=True)
    B, k1 = ot.shape
    k = k1 - 1
    for b in range(B):
        rep.rounds += 1
        rep.committed += int(gpu_nacc[b]) + 1
        gt, gn = gpu_tokens[b], int(gpu_nacc[b])
        if gn == on[b] and (gt == ot[b]).all():
            rep.exact += 1
            continue
        if not (0 <= gn <= k) or (gt[gn + 1:] != -1).any() or not (gt[:gn] == x[b, :gn]).all():
            rep.failures.append((b, "invalid round", gt.tolist(), ot[b].tolist()))
            continue
        if margin[b] < eps_trunc:
            rep.tie_trunc += 1
            continue
        t = tr[b]
        first = min(gn, int(on[b]))
        if gn != on[b]:
            if first < t.evaluated and t.accept_margin[first] < eps:
                rep.tie_accept += 1
            else:
                rep.failures.append((b, f"accepted length {gn} vs {on[b]}", gt.tolist(),
                                     ot[b].tolist(), t.accept_margin[first]))
            continue
        j = gn
        if t.sample_margin < eps and 0 <= gt[j] < z.shape[2]:
            lo, hi, w = _truncated_interval(z[b, j], y[b, j] if j < k else None, T, top_k, top_p,
                                            int(gt[j]))
            if w > 0 and lo - eps <= u[b, k] <= hi + eps:
                rep.tie_sample += 1
                continue
        rep.failures.append((b, f"drawn token {gt[j]} vs {ot[b, j]}", float(u[b, k]),
                             t.sample_lo, t.sample_hi, t.sample_margin))
    return rep


def check_probs_truncated(z, y, x, T, top_k, top_p, gpu_px, gpu_qx, eps_trunc=1e-5):
    """Largest relative error of the exported p'_i(x_i), q'_i(x_i) over the
    positions whose rows have a top-p margin of at least eps_trunc (the others
    may legitimately keep a different set); returns (worst, skipped rows)."""
    worst, skipped = 0.0, 0
    B, k = x.shape
    for b in range(B):
        for i in range(k):
            for row, got in ((z[b, i], gpu_px[b, i]), (y[b, i], gpu_qx[b, i])):
                p, m = truncated_row(row, T, top_k, top_p)
                if m < eps_trunc:
                    skipped += 1
                    continue
                ref = p[x[b, i]] if 0 <= x[b, i] < p.shape[0] else 0.0
                if ref == 0.0:
                    if got != 0.0:
                        return float("inf"), skipped
                    continue
                worst = max(worst, float(prob_error(got, ref)))
    return worst, skipped
