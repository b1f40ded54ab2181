"""Comparison of the GPU library's outputs with the CPU oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check).  Receives plain arrays; never
imports or calls the GPU library.

Greedy and candidate results must be bit-exact.  A sampling round must match
the oracle's round exactly, except where one of the oracle's own decisions
lies within `eps` of its boundary, where float32 rounding on the GPU may
legitimately go the other way.  Such a decision excuses that decision alone,
never the rest of the round:
  - an acceptance with |u_i - min(1, p/q)| < eps taken the other way: the
    oracle is run again on that sequence with u_i moved to the GPU's side
    (0 if the GPU accepted, the largest float32 below 1 if it rejected), and
    the GPU's round must match that run, by the same rules (so a later tie is
    handled the same way);
  - the round's draw with u_k within eps of a boundary of the drawn token's
    CDF interval: the GPU's token must be a token of positive weight whose own
    interval lies within eps of u_k;
  - truncated rows whose top-p boundary lies within eps_trunc of top_p (the
    oracle's trunc_margin): the GPU may keep the neighbouring set, so the
    round must match, by the rules above, the oracle run at top_p or at
    top_p -/+ eps_trunc, which keeps the neighbouring set of every such row.
Such rounds are counted, not hidden.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import (draw_interval, greedy, greedy_candidates, greedy_matches, row_argmax, sample,
               sample_lenient, sample_truncated, token_probs, truncated_row)

# the largest float32 below 1: a uniform that rejects every ratio below 1
U_BELOW_ONE = float(np.nextafter(np.float32(1.0), np.float32(0.0)))


@dataclasses.dataclass
class SampleReport:
    rounds: int = 0
    exact: int = 0
    tie_accept: int = 0
    tie_sample: int = 0
    tie_trunc: int = 0
    forced: int = 0                    # tied acceptance decisions forced the GPU's way
    failures: list = dataclasses.field(default_factory=list)
    committed: int = 0

    def ok(self):
        return not self.failures

    def count(self, kinds):
        """Counts a passing round by the first band it passed through."""
        if not kinds:
            self.exact += 1
        elif kinds[0] == "trunc":
            self.tie_trunc += 1
        elif kinds[0] == "accept":
            self.tie_accept += 1
        else:
            self.tie_sample += 1
        self.forced += kinds.count("accept")

    def summary(self):
        return (f"rounds={self.rounds} exact={self.exact} tie_accept={self.tie_accept} "
                f"tie_sample={self.tie_sample} tie_trunc={self.tie_trunc} forced={self.forced} "
                f"failures={len(self.failures)} "
                f"mean_committed={self.committed / max(1, self.rounds):.4f}")


def _draw_within(interval, j, token, u, eps, V):
    """The drawn `token` at row j has positive weight and its CDF interval
    lies within eps of u."""
    if not 0 <= token < V:
        return False
    lo, hi, w = interval(j, int(token))
    return w > 0 and lo - eps <= u <= hi + eps


def check_round(run, interval, u, gt, gn, V, eps):
    """One GPU round (tokens gt, accepted count gn) against the oracle on its
    sequence.  run(u) -> (tokens, num_accepted, trace) runs the oracle with
    the uniforms u [k+1]; interval(j, token) -> (lo, hi, weight) places a
    token in the distribution the round draws from at row j.  Returns
    (kinds, failure): the tie bands the round passed through, in order
    ("accept", "sample"), and None or a description of the mismatch."""
    ot, on, t = run(u)
    on = int(on)
    k = len(ot) - 1
    if gn == on and (gt == ot).all():
        return [], None
    first = min(gn, on)
    if not (0 <= gn <= k) or not (gt[:first] == ot[:first]).all():
        return [], ("accepted prefix differs", gt.tolist(), ot.tolist())
    if (gt[gn + 1:] != -1).any():
        return [], ("padding", gt.tolist(), ot.tolist())
    if gn != on:
        if not (first < t.evaluated and t.accept_margin[first] < eps):
            return [], (f"accepted length {gn} vs {on}", gt.tolist(), ot.tolist(),
                        t.accept_margin[first] if first < t.evaluated else None)
        gpu_accepts = gn > first
        u2 = np.array(u, dtype=np.float32, copy=True)
        u2[first] = 0.0 if gpu_accepts else U_BELOW_ONE
        _, on2, _ = run(u2)
        if (int(on2) > first) == gpu_accepts:
            kinds, fail = check_round(run, interval, u2, gt, gn, V, eps)
            return ["accept"] + kinds, fail
        # no uniform takes the oracle the GPU's way: its ratio is exactly 1
        # (the GPU rejected) or exactly 0 (the GPU accepted)
        if gpu_accepts:
            return [], (f"accepted at {first} where the oracle's ratio is 0", gt.tolist(), ot.tolist())
        # the GPU's round ends at `first` with a draw from that row's residual
        if _draw_within(interval, first, gt[first], float(u[k]), eps, V):
            return ["accept"], None
        return [], (f"draw at {first} after a forced rejection", gt.tolist(), float(u[k]))
    if t.sample_margin < eps and _draw_within(interval, gn, gt[gn], float(u[k]), eps, V):
        return ["sample"], None
    return [], (f"drawn token {gt[gn]} vs {ot[gn]}", float(u[k]), t.sample_lo, t.sample_hi,
                t.sample_margin)


def _one(a, b):
    return a[b:b + 1]


def check_sample(z, y, x, u, T, gpu_tokens, gpu_nacc, eps=1e-5, report=None,
                 seq_ids=None, lenience=None) -> SampleReport:
    """z [B,k+1,V], y [B,k,V] float32; x [B,k]; u [B,k+1]; GPU outputs as numpy.
    `lenience` (l >= 1) compares against the lenient rule instead."""
    rep = report or SampleReport()
    if lenience is None:
        ot, on, _ = sample(z, y, x, u, T, traces=True)
    else:
        ot, on, _ = sample_lenient(z, y, x, u, T, lenience, traces=True)
    B, k1 = ot.shape
    k = k1 - 1
    V = z.shape[2]
    for b in range(B):
        sid = b if seq_ids is None else seq_ids[b]
        rep.rounds += 1
        rep.committed += int(gpu_nacc[b]) + 1
        gt, gn = np.asarray(gpu_tokens[b]), int(gpu_nacc[b])
        if gn == on[b] and (gt == ot[b]).all():
            rep.exact += 1
            continue

        def run(uu, b=b):
            if lenience is None:
                a, n, tr = sample(_one(z, b), _one(y, b), _one(x, b), uu[None], T, traces=True)
            else:
                a, n, tr = sample_lenient(_one(z, b), _one(y, b), _one(x, b), uu[None], T, lenience,
                                          traces=True)
            return a[0], n[0], tr[0]

        def interval(j, tok, b=b):
            return draw_interval(z[b, j], y[b, j] if j < k else None, T, tok)

        kinds, fail = check_round(run, interval, u[b], gt, gn, V, eps)
        if fail is not None:
            rep.failures.append((sid,) + tuple(fail))
        else:
            rep.count(kinds)
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
                           eps_trunc=1e-5, report=None, seq_ids=None) -> SampleReport:
    """As check_sample, on top-k / top-p truncated rows.  A round in which some
    row's top-p boundary lies within eps_trunc of top_p (the oracle's
    trunc_margin) may keep a neighbouring set on the GPU: it must then match
    the oracle run at top_p - eps_trunc or top_p + eps_trunc, which keeps the
    neighbouring set of every such row (counted as tie_trunc)."""
    rep = report or SampleReport()
    ot, on, _, margin = sample_truncated(z, y, x, u, T, top_k, top_p, traces=True)
    B, k1 = ot.shape
    k = k1 - 1
    V = z.shape[2]
    for b in range(B):
        sid = b if seq_ids is None else seq_ids[b]
        rep.rounds += 1
        rep.committed += int(gpu_nacc[b]) + 1
        gt, gn = np.asarray(gpu_tokens[b]), int(gpu_nacc[b])
        if gn == on[b] and (gt == ot[b]).all():
            rep.exact += 1
            continue

        def against(tp, b=b):
            def run(uu):
                a, n, tr, _ = sample_truncated(_one(z, b), _one(y, b), _one(x, b), uu[None], T, top_k,
                                               tp, traces=True)
                return a[0], n[0], tr[0]

            def interval(j, tok):
                return _truncated_interval(z[b, j], y[b, j] if j < k else None, T, top_k, tp, tok)
            return check_round(run, interval, u[b], gt, gn, V, eps)

        kinds, fail = against(top_p)
        if fail is not None and margin[b] < eps_trunc:
            for tp in (top_p - eps_trunc, top_p + eps_trunc):
                if not tp > 0.0:
                    continue
                kinds2, fail2 = against(tp)
                if fail2 is None:
                    kinds, fail = ["trunc"] + kinds2, None
                    break
        if fail is not None:
            rep.failures.append((sid,) + tuple(fail))
        else:
            rep.count(kinds)
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
