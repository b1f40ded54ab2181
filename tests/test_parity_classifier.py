"""The sampling parity classifier (oracle/parity.py) on planted outcomes, on the CPU.

A tied decision (the oracle's |u - min(1, p/q)| or CDF-boundary distance
below 1e-5) excuses that decision only: the rest of the round must still be
what the rule does after it (production blog, "The acceptance rule": the
drafts are examined left to right, and the round ends with exactly one draw).
Each "GPU" outcome below is made by the oracle itself with the tied uniform
moved a little to the other side of its boundary, or on the neighbouring
top-p set; then single mistakes are planted after the tie, and the classifier
must catch every one of them.
"""
import numpy as np
import pytest

import oracle
from oracle import parity

EPS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _built():
    import os
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()


def softmax(v, T=1.0):
    a = np.asarray(v, np.float64) / T
    e = np.exp(a - a.max())
    return e / e.sum()


def chain(seed, B=1, k=6, V=40, T=1.0):
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, 1.5, (B, k + 1, V)).astype(np.float32)
    y = (z[:, :k] + rng.normal(0.0, 1.2, (B, k, V))).astype(np.float32)
    x = np.zeros((B, k), np.int32)
    for b in range(B):
        for i in range(k):
            x[b, i] = rng.choice(V, p=softmax(y[b, i], T))
    u = (rng.integers(0, 1 << 24, (B, k + 1)) / float(1 << 24)).astype(np.float32)
    return z, y, x, u


def ratio_at(z, y, x, i, T=1.0):
    p, q = oracle.token_probs(z[0], y[0], x[0], T)
    return min(1.0, p[i] / q[i]) if q[i] > 0 else 1.0


def tie_case(seed, gpu_accepts, want_next_ratio_below=None):
    """A round whose decision at position i sits 1e-8 from its boundary, and
    the round the oracle makes with that uniform 2e-6 on the other side (the
    "GPU" round).  Returns (z, y, x, u, i, gpu_tokens, gpu_nacc)."""
    for s in range(seed, seed + 500):
        z, y, x, u = chain(s)
        k = x.shape[1]
        for i in range(k - 1):
            r = ratio_at(z, y, x, i)
            if not 0.05 < r < 0.95:
                continue
            if want_next_ratio_below is not None and not ratio_at(z, y, x, i + 1) < want_next_ratio_below:
                continue
            u = u.copy()
            u[0, :i] = 0.0                             # every earlier draft accepted
            u[0, i] = np.float32(r)                    # the tie: |u - r| < 3e-8
            ot, on = oracle.sample(z, y, x, u, 1.0)
            oracle_accepts = on[0] > i
            if oracle_accepts == gpu_accepts:
                continue
            ug = u.copy()
            ug[0, i] = np.float32(r - 2e-6) if gpu_accepts else np.float32(r + 2e-6)
            gt, gn = oracle.sample(z, y, x, ug, 1.0)
            assert (gn[0] > i) == gpu_accepts
            return z, y, x, u, i, gt, gn
    raise AssertionError("no tie case found")


def classify(z, y, x, u, gt, gn):
    return parity.check_sample(z, y, x, u, 1.0, gt, gn, eps=EPS)


def far_token(z, y, j, u_k, exclude, k):
    """A token of positive weight whose CDF interval at row j is farther than
    1e-5 from u_k."""
    V = z.shape[2]
    for t in range(V):
        if t == exclude:
            continue
        lo, hi, w = oracle.draw_interval(z[0, j], y[0, j] if j < k else None, 1.0, t)
        if w > 0 and (u_k < lo - 1e-3 or u_k > hi + 1e-3):
            return t
    raise AssertionError("no far token")


@pytest.mark.parametrize("gpu_accepts", [True, False])
def test_tied_acceptance_passes(gpu_accepts):
    z, y, x, u, i, gt, gn = tie_case(100, gpu_accepts)
    rep = classify(z, y, x, u, gt, gn)
    assert rep.ok(), rep.failures
    assert rep.tie_accept == 1 and rep.forced >= 1


@pytest.mark.parametrize("gpu_accepts", [True, False])
def test_wrong_draw_after_a_tied_acceptance_fails(gpu_accepts):
    """The tie excuses the decision, not a wrong replacement or bonus token
    after it."""
    z, y, x, u, i, gt, gn = tie_case(200, gpu_accepts)
    k = x.shape[1]
    j = int(gn[0])
    bad = gt.copy()
    bad[0, j] = far_token(z, y, j, float(u[0, k]), int(gt[0, j]), k)
    rep = classify(z, y, x, u, bad, gn)
    assert not rep.ok() and rep.tie_accept == 0


def test_wrong_decision_after_a_tied_acceptance_fails():
    """After a tied acceptance the GPU also accepts the next draft, which the
    oracle clearly rejects (u far above its ratio): a failure."""
    z, y, x, u, i, _, _ = tie_case(300, True, want_next_ratio_below=0.9)
    u = u.copy()
    u[0, i + 1] = np.float32(0.999)
    ug = u.copy()
    ug[0, i] = 0.0                                     # the GPU's side of the tie ...
    ug[0, i + 1] = 0.0                                 # ... and a wrong acceptance after it
    gt, gn = oracle.sample(z, y, x, ug, 1.0)
    assert gn[0] >= i + 2
    rep = classify(z, y, x, u, gt, gn)
    assert not rep.ok()


def test_padding_after_a_tied_acceptance_fails():
    z, y, x, u, i, gt, gn = tie_case(400, False)
    k = x.shape[1]
    bad = gt.copy()
    j = int(gn[0])
    assert j < k
    bad[0, j + 1] = 0
    assert not classify(z, y, x, u, bad, gn).ok()


def ratio_one_case(seed):
    """A position whose ratio is exactly 1 (q(x) <= p(x)) with u the largest
    float32 below 1: the oracle accepts for every uniform, so a GPU that
    rejects there (its float32 ratio a hair below 1) cannot be matched by
    moving u; its draw from that row's residual is checked instead."""
    for s in range(seed, seed + 500):
        z, y, x, u = chain(s)
        k = x.shape[1]
        p, q = oracle.token_probs(z[0], y[0], x[0], 1.0)
        for i in range(k):
            if not q[i] <= p[i]:
                continue
            u = u.copy()
            u[0, :i] = 0.0
            u[0, i] = np.float32(parity.U_BELOW_ONE)
            _, on = oracle.sample(z, y, x, u, 1.0)
            assert on[0] > i
            u_k = float(u[0, k])
            tok = None
            for t in range(z.shape[2]):
                lo, hi, w = oracle.draw_interval(z[0, i], y[0, i], 1.0, t)
                if w > 0 and lo <= u_k < hi:
                    tok = t
            if tok is None:
                continue
            gt = np.full((1, k + 1), -1, np.int32)
            gt[0, :i] = x[0, :i]
            gt[0, i] = tok
            return z, y, x, u, i, gt, np.array([i], np.int32)
    raise AssertionError("no ratio-one case found")


def test_rejection_where_the_ratio_is_one():
    z, y, x, u, i, gt, gn = ratio_one_case(500)
    rep = classify(z, y, x, u, gt, gn)
    assert rep.ok(), rep.failures
    assert rep.tie_accept == 1
    bad = gt.copy()
    bad[0, i] = far_token(z, y, i, float(u[0, -1]), int(gt[0, i]), x.shape[1])
    assert not classify(z, y, x, u, bad, gn).ok()


def test_tied_draw():
    """u_k placed 1e-8 inside a token's CDF interval: the neighbouring token is
    accepted as a tie, a token far from u_k is not."""
    for s in range(600, 1100):
        z, y, x, u = chain(s)
        k = x.shape[1]
        ot, on = oracle.sample(z, y, x, u, 1.0)
        j = int(on[0])
        t = int(ot[0, j])
        lo, hi, w = oracle.draw_interval(z[0, j], y[0, j] if j < k else None, 1.0, t)
        nxt = next((v for v in range(t + 1, z.shape[2])
                    if oracle.draw_interval(z[0, j], y[0, j] if j < k else None, 1.0, v)[2] > 0), None)
        if nxt is None or hi - lo < 1e-4:
            continue
        u = u.copy()
        u[0, k] = np.float32(np.nextafter(np.float32(hi), np.float32(0)))
        ot, on = oracle.sample(z, y, x, u, 1.0)
        if ot[0, j] != t or on[0] != j:
            continue
        gt = ot.copy()
        gt[0, j] = nxt
        rep = classify(z, y, x, u, gt, on)
        assert rep.ok() and rep.tie_sample == 1, rep.failures
        gt[0, j] = far_token(z, y, j, float(u[0, k]), t, k)
        assert not classify(z, y, x, u, gt, on).ok()
        return
    raise AssertionError("no draw case found")


# ---------------------------------------------------------------------------
# truncated rows: the top-p boundary
# ---------------------------------------------------------------------------
def trunc_rows(delta):
    """A target row whose top-p boundary sits `delta` above top_p's group
    boundary (so the oracle keeps one more group than a GPU a hair below it
    would), and a draft row with no boundary near top_p."""
    z = np.array([1.9, 0.3, 1.4, -0.6, 0.9, -1.2, 0.1, 2.4, -0.2, -2.0], np.float32)
    y = np.array([1.5, 0.6, 1.2, -0.3, 1.1, -1.0, 0.0, 2.0, 0.2, -1.6], np.float32)
    p = softmax(z)
    cum = np.cumsum(np.sort(p)[::-1])
    top_p = float(cum[2]) + delta
    _, m = oracle.truncated_row(z, 1.0, 0, top_p)
    _, md = oracle.truncated_row(y, 1.0, 0, top_p)
    assert m < 2 * delta and md > 1e-3
    return z, y, top_p


def trunc_batch(B=400, k=3, seed=7):
    z1, y1, top_p = trunc_rows(1e-7)
    V = z1.shape[0]
    z = np.broadcast_to(z1, (B, k + 1, V)).copy()
    y = np.broadcast_to(y1, (B, k, V)).copy()
    rng = np.random.default_rng(seed)
    q, _ = oracle.truncated_row(y1, 1.0, 0, top_p)
    x = rng.choice(V, size=(B, k), p=q / q.sum()).astype(np.int32)
    u = (rng.integers(0, 1 << 24, (B, k + 1)) / float(1 << 24)).astype(np.float32)
    return z, y, x, u, top_p


def test_neighbouring_top_p_set_passes():
    z, y, x, u, top_p = trunc_batch()
    gt, gn = oracle.sample_truncated(z, y, x, u, 1.0, 0, top_p - 2e-7)   # the neighbouring set
    rep = parity.check_sample_truncated(z, y, x, u, 1.0, 0, top_p, gt, gn, eps=EPS)
    assert rep.ok(), rep.failures[:3]
    assert rep.tie_trunc > 0 and rep.exact + rep.tie_trunc + rep.tie_accept + rep.tie_sample == rep.rounds


def test_wrong_draw_under_a_top_p_tie_fails():
    """Rounds inside the top-p band are checked in full against the
    neighbouring set: a drawn token with no weight in either set, or a
    wrong accepted length, fails."""
    z, y, x, u, top_p = trunc_batch()
    ot, on = oracle.sample_truncated(z, y, x, u, 1.0, 0, top_p)
    gt, gn = oracle.sample_truncated(z, y, x, u, 1.0, 0, top_p - 2e-7)
    differ = np.nonzero((gn != on) | (gt != ot).any(axis=1))[0]
    assert differ.size > 0
    zero_w = int(np.argmin(z[0, 0]))                   # the lowest logit: dropped by both sets
    bad = gt.copy()
    b = differ[0]
    bad[b, gn[b]] = zero_w
    rep = parity.check_sample_truncated(z, y, x, u, 1.0, 0, top_p, bad, gn, eps=EPS)
    assert len(rep.failures) == 1 and rep.failures[0][0] == b
    # a round that commits one draft more than either set allows
    b = next(b for b in differ if gn[b] < x.shape[1])
    bad_t, bad_n = gt.copy(), gn.copy()
    bad_t[b, gn[b]] = x[b, gn[b]]
    bad_n[b] += 1
    bad_t[b, bad_n[b]] = 0
    rep = parity.check_sample_truncated(z, y, x, u, 1.0, 0, top_p, bad_t, bad_n, eps=EPS)
    assert len(rep.failures) == 1 and rep.failures[0][0] == b


def test_top_p_far_from_any_boundary_gets_no_band():
    """With top_p 1e-3 away from every boundary there is no band: a round made
    on another set fails."""
    z1, y1, top_p = trunc_rows(1e-3)
    z, y, x, u, _ = trunc_batch()
    gt, gn = oracle.sample_truncated(z, y, x, u, 1.0, 0, top_p - 2e-3)
    rep = parity.check_sample_truncated(z, y, x, u, 1.0, 0, top_p, gt, gn, eps=EPS)
    ot, on = oracle.sample_truncated(z, y, x, u, 1.0, 0, top_p)
    differ = int(((gn != on) | (gt != ot).any(axis=1)).sum())
    assert differ > 0 and len(rep.failures) == differ and rep.tie_trunc == 0
