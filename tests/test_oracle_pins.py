"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself or retypes its arithmetic: each
test checks a law, a printed value, a closed form or a special case, and the
planted-mistake variants of the oracle (``oracle.MUT_*``) show that the checks
have the power to catch the plausible mistakes.
"""
import os

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    oracle.lib()


def u24(rng, shape):
    return (rng.integers(0, 1 << 24, size=shape) / float(1 << 24)).astype(np.float32)


# ---------------------------------------------------------------------------
# Closed forms printed on the pages
# ---------------------------------------------------------------------------
def expected_tokens(a, k):
    # production blog, "Predicting the speedup": (1 - a^(k+1)) / (1 - a)
    return (1 - a ** (k + 1)) / (1 - a)


def pgf_coefficients(a, k):
    """Coefficients of phi(x) = 1 + (x-1)(1 - a^(k+1) x^(k+1))/(1 - a x)
    (Cascade Speculative Drafting, Theorem 4.1), expanded by polynomial algebra:
    (1 - (ax)^(k+1))/(1 - ax) is the finite geometric sum of (ax)^j, j <= k."""
    geo = np.array([a ** j for j in range(k + 1)])
    poly = np.zeros(k + 2)
    poly[0] += 1.0
    poly[1:] += geo          # x * geo
    poly[:-1] -= geo         # -1 * geo
    return poly


def test_golden_blog_values():
    """The closed forms reproduce every number the blog prints."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "blog_expected_tokens.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 5
    for kind, a, k, c, val, dec in rows:
        a, k, val, dec = float(a), int(k), float(val), int(dec)
        e = expected_tokens(a, k)
        got = e if kind == "expected_tokens" else e / (k * float(c) + 1)
        assert round(got, dec) == pytest.approx(val), (kind, a, k, got, val)


@pytest.mark.parametrize("a,k", [(0.8, 4), (0.6, 4), (0.39, 16), (0.5, 1)])
def test_pgf_expansion_matches_printed_coefficients(a, k):
    """Theorem 4.1 of the Cascade page: the x^i coefficient is a^(i-1) - a^i
    for 1 <= i <= k and a^k for i = k+1; phi'(1) is the blog's expected value.
    The coefficient of x^i is read as P(i tokens committed in the round)."""
    c = pgf_coefficients(a, k)
    assert abs(c[0]) < 1e-15
    for i in range(1, k + 1):
        assert c[i] == pytest.approx(a ** (i - 1) - a ** i, abs=1e-14)
    assert c[k + 1] == pytest.approx(a ** k, abs=1e-14)
    assert c.sum() == pytest.approx(1.0, abs=1e-14)
    assert (np.arange(k + 2) * c).sum() == pytest.approx(expected_tokens(a, k), abs=1e-12)


def iid_acceptance_rows(a, rng):
    """V = 8.  m: a mixture over tokens 0..5.  p = a m + (1-a) e7, q = a m + (1-a) e6.
    A draft x ~ q is then accepted with certainty when x < 6 (p = q there) and
    never when x = 6 (p = 0), so acceptance is Bernoulli(a), independently per
    position, and sum_v min(p_v, q_v) = a."""
    m = rng.dirichlet(np.ones(6))
    p = np.zeros(8)
    q = np.zeros(8)
    p[:6] = a * m
    q[:6] = a * m
    p[7] = 1 - a
    q[6] = 1 - a
    with np.errstate(divide="ignore"):
        return np.log(p).astype(np.float32), np.log(q).astype(np.float32), q


def run_iid_rounds(a, k, n, seed, mutation=oracle.MUT_NONE):
    rng = np.random.default_rng(seed)
    zl, yl, q = iid_acceptance_rows(a, rng)
    z = np.broadcast_to(zl, (n, k + 1, 8)).copy()
    y = np.broadcast_to(yl, (n, k, 8)).copy()
    x = rng.choice(8, size=(n, k), p=q / q.sum()).astype(np.int32)
    u = u24(rng, (n, k + 1))
    _, na = oracle.sample(z, y, x, u, 1.0, mutation=mutation)
    return na + 1  # committed tokens per round


@pytest.mark.parametrize("a,k", [(0.8, 4), (0.6, 4)])
def test_iid_acceptance_mean_and_law(a, k):
    """Mean committed tokens per round = (1 - a^(k+1))/(1 - a) (blog: 3.36 at
    a = 0.8, 2.31 at a = 0.6, k = 4) within 4 standard errors, and the full
    committed-count histogram follows the Theorem 4.1 coefficients."""
    n = 200_000
    committed = run_iid_rounds(a, k, n, seed=11)
    coef = pgf_coefficients(a, k)[1:]
    mean = (np.arange(1, k + 2) * coef).sum()
    sd = np.sqrt((np.arange(1, k + 2) ** 2 * coef).sum() - mean ** 2)
    assert abs(committed.mean() - expected_tokens(a, k)) < 4 * sd / np.sqrt(n)
    hist = np.bincount(committed, minlength=k + 2)[1:]
    chi = scipy.stats.chisquare(hist, coef * n)
    assert chi.pvalue > 1e-4, (hist, coef * n)


def test_iid_acceptance_detects_inverted_ratio():
    committed = run_iid_rounds(0.8, 4, 50_000, seed=12, mutation=oracle.MUT_RATIO_INVERTED)
    assert abs(committed.mean() - expected_tokens(0.8, 4)) > 0.2


# ---------------------------------------------------------------------------
# Exact law of the committed tokens at V = 8 (brute force over the draft token
# and exact integration over the uniforms by bisection on the 2^-24 grid)
# ---------------------------------------------------------------------------
GRID = 1 << 24


class Probe:
    """Calls the oracle on one fixed set of rows with many uniform vectors."""

    def __init__(self, P, Q, T, mutation, lenience=None):
        self.lenience = lenience
        self.k = Q.shape[0]
        V = P.shape[1]
        with np.errstate(divide="ignore"):
            self.z = (T * np.log(P)).astype(np.float32)
            self.y = (T * np.log(Q)).astype(np.float32)
        self.T = T
        self.mut = mutation
        self.V = V

    def run(self, x, U):
        n = U.shape[0]
        z = np.broadcast_to(self.z, (n,) + self.z.shape).copy()
        y = np.broadcast_to(self.y, (n,) + self.y.shape).copy()
        xx = np.broadcast_to(np.asarray(x, np.int32), (n, self.k)).copy()
        if self.lenience is not None:
            return oracle.sample_lenient(z, y, xx, U.astype(np.float32), self.T, self.lenience)
        return oracle.sample(z, y, xx, U.astype(np.float32), self.T, mutation=self.mut)

    def measure(self, x, base_u, coord, pred):
        """Number of grid points g in [0, 2^24) with pred(out(u[coord] = g/2^24))
        true, for predicates that hold on an initial segment; vectorised over a
        batch of predicates (pred returns a bool array over the batch)."""
        npred = pred(None)
        lo = np.zeros(npred, np.int64)
        hi = np.full(npred, GRID, np.int64)
        while np.any(lo < hi):
            mid = (lo + hi) // 2
            U = np.broadcast_to(base_u, (npred, base_u.size)).copy()
            U[:, coord] = mid / GRID
            tokens, na = self.run(x, U)
            ok = pred((tokens, na))
            act = lo < hi
            lo = np.where(act & ok, mid + 1, lo)
            hi = np.where(act & ~ok, mid, hi)
        return lo / GRID


def committed_law(P, Q, T, mutation=oracle.MUT_NONE, lenience=None):
    """Exact law (on the uniform grid) of the token committed at each position i,
    given that the round reaches i, and the acceptance probability at i."""
    k, V = Q.shape
    pr = Probe(P, Q, T, mutation, lenience)
    # a draft that is surely accepted with u = 0 (p > 0 there) for the prefix
    safe = [int(np.argmax(np.minimum(P[i], Q[i]) + 1e-3 * (P[i] > 0))) for i in range(k)]
    laws, acc = [], []
    for i in range(k):
        law = np.zeros(V)
        a_tot = 0.0
        for xv in range(V):
            if Q[i, xv] == 0:
                continue
            x = safe.copy()
            x[i] = xv
            base = np.zeros(k + 1)
            a = pr.measure(x, base, i, lambda r: 1 if r is None else (r[1] > i))[0]
            a_tot += Q[i, xv] * a
            law[xv] += Q[i, xv] * a
            if a < 1.0:
                base[i] = a          # the first grid point that rejects
                cdf = pr.measure(x, base, k,
                                 lambda r: V if r is None else (r[0][:, i] <= np.arange(V)))
                law += Q[i, xv] * (1 - a) * np.diff(np.concatenate([[0.0], cdf]))
        laws.append(law)
        acc.append(a_tot)
    # bonus: every draft accepted
    x = safe.copy()
    base = np.zeros(k + 1)
    cdf = pr.measure(x, base, k, lambda r: V if r is None else (r[0][:, k] <= np.arange(V)))
    assert all(P[i, safe[i]] > 0 for i in range(k))
    laws.append(np.diff(np.concatenate([[0.0], cdf])))
    return np.array(laws), np.array(acc)


def v8_cases():
    rng = np.random.default_rng(5)
    k = 3
    cases = []
    # generic: full support
    cases.append(("dirichlet", rng.dirichlet(np.ones(8), k + 1), rng.dirichlet(np.ones(8), k), 1.0))
    # temperature other than 1, uneven distributions
    cases.append(("peaked_T0.7", rng.dirichlet(0.3 * np.ones(8), k + 1),
                  rng.dirichlet(0.3 * np.ones(8), k), 0.7))
    # masked tokens (zero probability, logit -inf) on both sides
    P = rng.dirichlet(np.ones(8), k + 1)
    Q = rng.dirichlet(np.ones(8), k)
    P[:, [1, 5]] = 0
    Q[:, [2, 5]] = 0
    P /= P.sum(1, keepdims=True)
    Q /= Q.sum(1, keepdims=True)
    cases.append(("masked_T1.6", P, Q, 1.6))
    # disjoint supports: every draft is rejected, the residual is p
    P = np.zeros((k + 1, 8))
    Q = np.zeros((k, 8))
    P[:, :4] = rng.dirichlet(np.ones(4), k + 1)
    Q[:, 4:] = rng.dirichlet(np.ones(4), k)
    cases.append(("disjoint", P, Q, 1.0))
    return cases


@pytest.mark.parametrize("name,P,Q,T", v8_cases(), ids=lambda v: v if isinstance(v, str) else "")
def test_v8_committed_token_is_target_distributed(name, P, Q, T):
    """Blog, "The acceptance rule": every committed token is distributed exactly
    as a sample from the target; the acceptance probability at a position is
    sum_v min(p_v, q_v) (the standard identity for x ~ q kept w.p. min(1, p/q))."""
    laws, acc = committed_law(P, Q, T)
    k = Q.shape[0]
    for i in range(k + 1):
        np.testing.assert_allclose(laws[i], P[i], atol=2e-6, err_msg=f"{name} position {i}")
    np.testing.assert_allclose(acc, np.minimum(P[:k], Q).sum(1), atol=2e-6)


@pytest.mark.parametrize("mutation", [oracle.MUT_RESIDUAL_IS_P, oracle.MUT_RESIDUAL_IS_Q,
                                      oracle.MUT_BONUS_FROM_Q, oracle.MUT_RATIO_INVERTED,
                                      oracle.MUT_RESIDUAL_SIGN])
def test_v8_law_catches_planted_mistakes(mutation):
    name, P, Q, T = v8_cases()[0]
    laws, acc = committed_law(P, Q, T, mutation)
    k = Q.shape[0]
    dev = max(np.abs(laws - P).max(), np.abs(acc - np.minimum(P[:k], Q).sum(1)).max())
    assert dev > 1e-2, dev


# ---------------------------------------------------------------------------
# Histogram test with and without speculation (blog: compare token histograms
# of continuations sampled with and without speculation)
# ---------------------------------------------------------------------------
def merged_two_sample_pvalue(a, b, V, min_pooled=40):
    ca = np.bincount(a, minlength=V).astype(np.float64)
    cb = np.bincount(b, minlength=V).astype(np.float64)
    order = np.argsort(-(ca + cb), kind="stable")
    groups_a, groups_b = [], []
    acc_a = acc_b = 0.0
    for t in order:
        acc_a += ca[t]
        acc_b += cb[t]
        if acc_a + acc_b >= min_pooled:
            groups_a.append(acc_a)
            groups_b.append(acc_b)
            acc_a = acc_b = 0.0
    if acc_a + acc_b > 0 and groups_a:
        groups_a[-1] += acc_a
        groups_b[-1] += acc_b
    table = np.array([groups_a, groups_b])
    return scipy.stats.chi2_contingency(table)[1]


def histogram_experiment(mutation, n=60_000, V=500, k=3, T=1.0, seed=21):
    g = torch.Generator().manual_seed(seed)
    z = torch.randn((k + 1, V), generator=g) * np.sqrt(2.0)
    y = z[:k] + torch.randn((k, V), generator=g)
    rng = np.random.default_rng(seed)
    # without speculation: direct draws from each target row
    direct = [synthetic.gumbel_max_sample(z[i:i + 1].expand(n, V), T, g).numpy() for i in range(k + 1)]
    toks, nas = [], []
    chunk = 4096
    zz = z.numpy().astype(np.float32)
    yy = y.numpy().astype(np.float32)
    for s0 in range(0, n, chunk):
        m = min(chunk, n - s0)
        x = torch.stack([synthetic.gumbel_max_sample(y[i:i + 1].expand(m, V), T, g)
                         for i in range(k)], dim=1).numpy()
        u = u24(rng, (m, k + 1))
        t, na = oracle.sample(np.broadcast_to(zz, (m, k + 1, V)).copy(),
                              np.broadcast_to(yy, (m, k, V)).copy(), x, u, T, mutation=mutation)
        toks.append(t)
        nas.append(na)
    toks = np.concatenate(toks)
    nas = np.concatenate(nas)
    pvals = []
    for i in (0, 1, k):
        reach = nas >= i
        pvals.append(merged_two_sample_pvalue(toks[reach, i], direct[i][: reach.sum()], V))
    return pvals, nas


def test_histogram_with_and_without_speculation():
    pvals, nas = histogram_experiment(oracle.MUT_NONE)
    assert (nas == 3).sum() > 3000   # the bonus position is reached often enough
    assert min(pvals) > 1e-4, pvals


@pytest.mark.parametrize("mutation", [oracle.MUT_RESIDUAL_IS_P, oracle.MUT_RESIDUAL_IS_Q,
                                      oracle.MUT_BONUS_FROM_Q, oracle.MUT_RESIDUAL_SIGN])
def test_histogram_catches_planted_mistakes(mutation):
    pvals, _ = histogram_experiment(mutation, n=30_000)
    assert min(pvals) < 1e-6, pvals


def softmax64(v, T=1.0):
    a = np.asarray(v, np.float64) / T
    e = np.exp(a - a.max())
    return e / e.sum()


def merged_gof_pvalue(tokens, p, min_expected=20.0):
    """Chi-square goodness of fit of `tokens` against the distribution p, the
    tokens taken in descending order of p and merged into bins whose expected
    count reaches `min_expected` (the rest joins the last bin)."""
    n = tokens.size
    counts = np.bincount(tokens, minlength=p.size).astype(np.float64)
    order = np.argsort(-p, kind="stable")
    obs, exp_ = [], []
    o = e = 0.0
    for t in order:
        o += counts[t]
        e += n * p[t]
        if e >= min_expected:
            obs.append(o)
            exp_.append(e)
            o = e = 0.0
    obs[-1] += o
    exp_[-1] += e
    obs, exp_ = np.array(obs), np.array(exp_)
    stat = ((obs - exp_) ** 2 / exp_).sum()
    return scipy.stats.chi2.sf(stat, obs.size - 1)


def histogram_experiment_workload1_shape(mutation, n, seed=31, chunk=128):
    """Rounds at workload 1's shape (k = 4, V = 32000, target logits N(0, var
    2), draft = target + N(0, var 1), T = 1): the draft tokens drawn from q
    (numpy's sampler), uniforms on the 2^-24 grid, the oracle run on 8
    threads.  Returns the p-values, at positions 0, 1 and k, of the
    committed tokens (rounds that reach the position) against direct draws
    from p (two-sample) and against p itself (goodness of fit), and the
    accepted counts."""
    import concurrent.futures
    V, k, T = 32000, 4, 1.0
    rng = np.random.default_rng(seed)
    z = rng.normal(0.0, np.sqrt(2.0), (k + 1, V)).astype(np.float32)
    y = (z[:k] + rng.normal(0.0, 1.0, (k, V))).astype(np.float32)
    p = [softmax64(z[i], T) for i in range(k + 1)]
    q = [softmax64(y[i], T) for i in range(k)]
    x = np.stack([rng.choice(V, size=n, p=q[i]) for i in range(k)], axis=1).astype(np.int32)
    u = u24(rng, (n, k + 1))

    def run(s0):
        m = min(chunk, n - s0)
        return oracle.sample(np.broadcast_to(z, (m, k + 1, V)).copy(), np.broadcast_to(y, (m, k, V)).copy(),
                             x[s0:s0 + m], u[s0:s0 + m], T, mutation=mutation)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(run, range(0, n, chunk)))
    toks = np.concatenate([t for t, _ in parts])
    nas = np.concatenate([a for _, a in parts])
    pvals = []
    for i in (0, 1, k):
        got = toks[nas >= i, i]
        direct = rng.choice(V, size=got.size, p=p[i])      # without speculation
        pvals.append(merged_two_sample_pvalue(got, direct, V))
        pvals.append(merged_gof_pvalue(got, p[i]))
    return pvals, nas


def test_histogram_at_the_workload_1_shape():
    """The Blog's advice (compare token histograms with and without
    speculation) at workload 1's vocabulary of 32000: 32000 rounds, the
    committed token at positions 0, 1 and k against direct draws from the
    target's p and against p itself, bins merged to expected counts of at
    least 20."""
    pvals, nas = histogram_experiment_workload1_shape(oracle.MUT_NONE, n=32_000)
    assert (nas == 4).sum() > 3000          # the bonus position is reached often enough
    assert min(pvals) > 1e-4, pvals


@pytest.mark.parametrize("mutation", [oracle.MUT_RESIDUAL_IS_P, oracle.MUT_RESIDUAL_IS_Q,
                                      oracle.MUT_BONUS_FROM_Q, oracle.MUT_RESIDUAL_SIGN])
def test_histogram_at_the_workload_1_shape_catches_planted_mistakes(mutation):
    pvals, _ = histogram_experiment_workload1_shape(mutation, n=12_000)
    assert min(pvals) < 1e-6, pvals


# ---------------------------------------------------------------------------
# Special cases
# ---------------------------------------------------------------------------
def test_one_hot_rows_sampling_equals_greedy():
    """Greedy collapse (blog, end of "The acceptance rule"; Double, D.2: with
    T = 0 replacing a rejected draft by the target token is residual sampling):
    with one-hot p and q the sampling rule gives the greedy result for any u."""
    rng = np.random.default_rng(3)
    n, k, V = 4000, 5, 16
    ta = rng.integers(0, V, (n, k + 1))
    xa = np.where(rng.random((n, k)) < 0.7, ta[:, :k], rng.integers(0, V, (n, k)))
    z = np.full((n, k + 1, V), -np.inf, np.float32)
    y = np.full((n, k, V), -np.inf, np.float32)
    np.put_along_axis(z, ta[..., None], 0.0, axis=2)
    np.put_along_axis(y, xa[..., None], 0.0, axis=2)
    u = u24(rng, (n, k + 1))
    ts, ns = oracle.sample(z, y, xa, u, 1.0)
    tg, ng = oracle.greedy(z, xa)
    np.testing.assert_array_equal(ns, ng)
    np.testing.assert_array_equal(ts, tg)


def test_low_temperature_sampling_equals_greedy():
    """The T -> 0 limit of the sampling rule is the greedy rule."""
    rng = np.random.default_rng(4)
    n, k, V = 500, 4, 64
    z = rng.integers(-20, 20, (n, k + 1, V)).astype(np.float32)
    y = rng.integers(-20, 20, (n, k, V)).astype(np.float32)
    # unique maxima, a margin of 1 above the rest
    tz = rng.integers(0, V, (n, k + 1))
    ty = np.where(rng.random((n, k)) < 0.6, tz[:, :k], rng.integers(0, V, (n, k)))
    np.put_along_axis(z, tz[..., None], 21.0, axis=2)
    np.put_along_axis(y, ty[..., None], 21.0, axis=2)
    x = ty.astype(np.int32)          # the draft's (almost sure) sample
    u = np.clip(u24(rng, (n, k + 1)), 1e-3, 1 - 1e-3).astype(np.float32)
    ts, ns = oracle.sample(z, y, x, u, 0.01)
    tg, ng = oracle.greedy(z, x)
    np.testing.assert_array_equal(ns, ng)
    np.testing.assert_array_equal(ts, tg)


def test_identical_target_and_draft_accepts_everything():
    rng = np.random.default_rng(6)
    n, k, V = 300, 6, 50
    z = rng.normal(0, 2, (n, k + 1, V)).astype(np.float32)
    y = z[:, :k].copy()
    x = rng.integers(0, V, (n, k)).astype(np.int32)
    u = u24(rng, (n, k + 1))
    t, na = oracle.sample(z, y, x, u, 0.8)
    assert (na == k).all()
    np.testing.assert_array_equal(t[:, :k], x)
    assert ((t[:, k] >= 0) & (t[:, k] < V)).all()


def test_invalid_draft_token_is_rejected():
    rng = np.random.default_rng(7)
    n, k, V = 200, 4, 32
    z = rng.normal(0, 1, (n, k + 1, V)).astype(np.float32)
    y = z[:, :k].copy()                  # p = q: every valid token is accepted
    x = np.argmax(z[:, :k], axis=2).astype(np.int32)   # and greedy accepts these
    pos = rng.integers(0, k, n)
    bad = np.where(rng.random(n) < 0.5, -1 - rng.integers(0, 5, n), V + rng.integers(0, 5, n))
    x[np.arange(n), pos] = bad
    u = u24(rng, (n, k + 1))
    t, na = oracle.sample(z, y, x, u, 1.0)
    np.testing.assert_array_equal(na, pos)
    tg, ng = oracle.greedy(z, x)
    np.testing.assert_array_equal(ng, pos)
    assert ((t[np.arange(n), pos] >= 0) & (t[np.arange(n), pos] < V)).all()


def test_greedy_argmax_is_first_maximum():
    """Greedy against numpy's first-occurrence argmax on tie-heavy rows,
    including -0.0 / +0.0 ties, all -inf rows (index 0) and NaN entries."""
    rng = np.random.default_rng(8)
    n, k, V = 2000, 3, 40
    z = rng.integers(-3, 3, (n, k + 1, V)).astype(np.float32)
    z[z == 0] = np.where(rng.random((z == 0).sum()) < 0.5, -0.0, 0.0)
    z[::17] = -np.inf
    nan_mask = rng.random(z.shape) < 0.02
    z[nan_mask] = np.nan
    ref = np.argmax(np.where(np.isnan(z), -np.inf, z), axis=2)
    # drafts: the reference argmax at a random number of leading positions
    j = rng.integers(0, k + 1, n)
    x = rng.integers(0, V, (n, k))
    for b in range(n):
        x[b, :j[b]] = ref[b, :j[b]]
    t, na = oracle.greedy(z, x.astype(np.int32))
    for b in range(n):
        jb = 0
        while jb < k and x[b, jb] == ref[b, jb]:
            jb += 1
        assert na[b] == jb
        exp = list(x[b, :jb]) + [ref[b, jb]] + [-1] * (k - jb)
        np.testing.assert_array_equal(t[b], exp)


def test_residual_mass_zero_falls_back_to_target():
    """A rejection needs p(x) < q(x), and then some token has p > q, so the
    residual total S is positive in exact arithmetic (the S = 0 reading, sample
    from p, only guards rounding).  Every rejection here samples the residual and
    every full acceptance the bonus row."""
    rng = np.random.default_rng(9)
    n, k, V = 2000, 3, 12
    z = rng.normal(0, 1, (n, k + 1, V)).astype(np.float32)
    y = (z[:, :k] + rng.normal(0, 1, (n, k, V))).astype(np.float32)
    x = rng.integers(0, V, (n, k)).astype(np.int32)
    u = u24(rng, (n, k + 1))
    _, na, tr = oracle.sample(z, y, x, u, 1.0, traces=True)
    kinds = np.array([t.sample_kind for t in tr])
    assert set(kinds[na < k]) == {0}
    assert set(kinds[na == k]) <= {1}


# ---------------------------------------------------------------------------
# Multi-candidate selection
# ---------------------------------------------------------------------------
def candidates_closed_form(a, C, L, prefix):
    """E[A] when every token independently equals its row's argmax w.p. a, the
    first `prefix` tokens shared by all C candidates: P(A >= n) = a^n for
    n <= prefix, a^prefix (1 - (1 - a^(n - prefix))^C) beyond."""
    e = 0.0
    for n in range(1, L + 1):
        if n <= prefix:
            e += a ** n
        else:
            e += a ** prefix * (1 - (1 - a ** (n - prefix)) ** C)
    return e


def test_candidates_closed_form_expected_length():
    assert candidates_closed_form(0.8, 8, 8, 2) == pytest.approx(5.18537, abs=1e-5)
    rng = np.random.default_rng(10)
    B, C, L, V = 20000, 8, 8, 16
    R = L
    z = rng.normal(0, 1, (B, C, R, V)).astype(np.float32)
    spikes = rng.integers(0, V, (B, C, R))
    spikes[:, :, :3] = spikes[:, :1, :3]
    z[:, :, :3] = z[:, :1, :3]
    np.put_along_axis(z, spikes[..., None], 100.0, axis=3)   # the argmax by construction
    hit = rng.random((B, C, L)) < 0.8
    other = (spikes[:, :, :L] + rng.integers(1, V, (B, C, L))) % V
    cand = np.where(hit, spikes[:, :, :L], other)
    cand[:, :, :2] = cand[:, :1, :2]
    out, A, best = oracle.greedy_candidates(z, cand.astype(np.int32))
    e = candidates_closed_form(0.8, C, L, 2)
    assert abs(A.mean() - e) < 4 * A.std() / np.sqrt(B)


def test_candidates_selection_properties():
    """Ouroboros 3.4.3 selection: the committed prefix is the chosen candidate's
    accepted tokens, no candidate has a longer accepted run, ties go to the lowest
    candidate index, and the correction is the argmax at the first mismatch."""
    rng = np.random.default_rng(11)
    B, C, L, V = 3000, 4, 5, 6
    for R in (L, L + 1):
        z = rng.integers(0, 4, (B, C, R, V)).astype(np.float32)
        ref = np.argmax(z, axis=3)
        cand = np.where(rng.random((B, C, L)) < 0.75, ref[:, :, :L], rng.integers(0, V, (B, C, L)))
        out, A, best = oracle.greedy_candidates(z, cand.astype(np.int32))
        for b in range(B):
            runs = []
            for c in range(C):
                a = 0
                while a < L and cand[b, c, a] == ref[b, c, a]:
                    a += 1
                runs.append(a)
            assert A[b] == max(runs)
            assert best[b] == runs.index(max(runs))
            cs = best[b]
            np.testing.assert_array_equal(out[b, :A[b]], cand[b, cs, :A[b]])
            if A[b] < L:
                assert out[b, A[b]] == ref[b, cs, A[b]]
                assert (out[b, A[b] + 1:] == -1).all()
            elif R == L + 1:
                assert out[b, L] == ref[b, cs, L]
            else:
                assert out[b, L] == -1


# ---------------------------------------------------------------------------
# Lenience (Cascade Speculative Drafting, "The Vertical Cascade": accept if
# q <= l p, else reject with probability 1 - l p / q; residual max(0, p - q))
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lenience", [1.5, 4.0])
def test_v8_lenient_law(lenience):
    """With x ~ q kept w.p. min(1, l p/q), a position accepts with probability
    sum_v min(q_v, l p_v), and commits v with probability
    min(q_v, l p_v) + (1 - sum_w min(q_w, l p_w)) r_v / sum r, r = max(0, p - q)."""
    name, P, Q, T = v8_cases()[1]
    laws, acc = committed_law(P, Q, T, lenience=lenience)
    k = Q.shape[0]
    for i in range(k):
        a = np.minimum(Q[i], lenience * P[i])
        r = np.maximum(P[i] - Q[i], 0.0)
        expect = a + (1 - a.sum()) * r / r.sum()
        np.testing.assert_allclose(laws[i], expect, atol=3e-6, err_msg=f"position {i}")
        assert acc[i] == pytest.approx(a.sum(), abs=3e-6)
    np.testing.assert_allclose(laws[k], P[k], atol=3e-6)
    # lenience moves mass toward q: the law is no longer p
    assert np.abs(laws[:k] - P[:k]).max() > 1e-2


def test_lenience_one_is_the_rule_and_large_lenience_accepts_all():
    rng = np.random.default_rng(13)
    n, k, V = 400, 5, 64
    z = rng.normal(0, 1.5, (n, k + 1, V)).astype(np.float32)
    y = (z[:, :k] + rng.normal(0, 1.5, (n, k, V))).astype(np.float32)
    x = rng.integers(0, V, (n, k)).astype(np.int32)
    u = u24(rng, (n, k + 1))
    t1, n1 = oracle.sample(z, y, x, u, 0.9)
    t2, n2 = oracle.sample_lenient(z, y, x, u, 0.9, 1.0)
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_array_equal(n1, n2)
    # l = 1e30: every finite-logit draft passes q <= l p
    t3, n3 = oracle.sample_lenient(z, y, x, u, 0.9, 1e30)
    assert (n3 == k).all()
    np.testing.assert_array_equal(t3[:, :k], x)


# ---------------------------------------------------------------------------
# #Match (Ouroboros section 3.4.4, Eq. 10)
# ---------------------------------------------------------------------------
def test_greedy_matches_definition_and_bound():
    """v_i is the first-occurrence argmax of row i (numpy, independently of the
    oracle), the mask marks x_i == v_i, #Match is its popcount, and #Match is at
    least the accepted length A, with equality when the rejected tail has no
    match (the page: #Match is always at least A)."""
    rng = np.random.default_rng(14)
    n, k, V = 3000, 7, 30
    z = rng.integers(-4, 4, (n, k + 1, V)).astype(np.float32)
    ref = np.argmax(z, axis=2)
    x = np.where(rng.random((n, k)) < 0.6, ref[:, :k], rng.integers(0, V, (n, k))).astype(np.int32)
    v, mask, cnt = oracle.greedy_matches(z, x)
    np.testing.assert_array_equal(v, ref)
    bits = (x == ref[:, :k])
    want_mask = (bits * (1 << np.arange(k))).sum(axis=1).astype(np.uint64)
    np.testing.assert_array_equal(mask, want_mask)
    np.testing.assert_array_equal(cnt, bits.sum(axis=1))
    _, A = oracle.greedy(z, x)
    assert (cnt >= A).all()
    tail_match = np.array([bits[b, A[b] + 1:].any() if A[b] < k else False for b in range(n)])
    np.testing.assert_array_equal(cnt == A, ~tail_match)
    # the committed tokens are v up to and including the first mismatch
    toks, _ = oracle.greedy(z, x)
    for b in range(0, n, 97):
        np.testing.assert_array_equal(toks[b, : A[b] + 1], v[b, : A[b] + 1])


def test_row_argmax_matches_numpy():
    rng = np.random.default_rng(15)
    z = rng.integers(-3, 3, (50, 7, 41)).astype(np.float32)
    np.testing.assert_array_equal(oracle.row_argmax(z), np.argmax(z, axis=2))


# ---------------------------------------------------------------------------
# Token tree (Ouroboros 3.4.3, Figure 3): the tree is the flat candidate
# layout with shared rows stored once
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("R_extra", [0, 1])
def test_tree_equals_flat_layout(R_extra):
    """Spelling every candidate's rows out of the tree gives the flat layout;
    the tree selection must equal the (pinned) flat selection on it."""
    rng = np.random.default_rng(16)
    B, C, L, V, S = 400, 5, 6, 12, 3
    R = L + R_extra
    N = S + C * (R - S)
    nodes = rng.integers(-3, 3, (B, N, V)).astype(np.float32)
    rows = np.zeros((B, C, R), np.int32)
    for c in range(C):
        rows[:, c, :S] = np.arange(S)
        rows[:, c, S:] = S + c * (R - S) + np.arange(R - S)
    flat = np.take_along_axis(nodes[:, None, :, :], rows[..., None].astype(np.int64), axis=2)
    ref = np.argmax(flat, axis=3)
    cand = np.where(rng.random((B, C, L)) < 0.8, ref[:, :, :L], rng.integers(0, V, (B, C, L)))
    cand[:, :, :S - 1] = cand[:, :1, :S - 1]
    t1, a1, b1 = oracle.greedy_tree(nodes, cand, rows)
    t2, a2, b2 = oracle.greedy_candidates(flat, cand)
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(b1, b2)


def test_tree_invalid_row_index_never_matches():
    rng = np.random.default_rng(17)
    B, C, L, V, N = 50, 2, 3, 9, 6
    nodes = rng.normal(size=(B, N, V)).astype(np.float32)
    rows = rng.integers(0, N, (B, C, L)).astype(np.int32)
    ref = np.argmax(np.take_along_axis(nodes[:, None], rows[..., None].astype(np.int64), axis=2), axis=3)
    cand = ref.copy()                                   # everything matches ...
    rows[:, 1, 1] = N + 3                               # ... except where the row is invalid
    rows[:, 0, 2] = -1
    t, a, best = oracle.greedy_tree(nodes, cand, rows)
    assert (a == 2).all() and (best == 0).all()
    assert (t[:, 2] == -1).all()                        # correction from an invalid row


def test_tree_padding_slots_never_match():
    """A tree builder that pads a short candidate with token -1 at row -1 gets
    nothing from the padding: a row outside [0, N) scores nothing, so its
    position is a mismatch whatever the token (the -1 token included)."""
    rng = np.random.default_rng(19)
    B, C, L, V, N = 40, 3, 4, 11, 7
    nodes = rng.normal(size=(B, N, V)).astype(np.float32)
    rows = rng.integers(0, N, (B, C, L)).astype(np.int32)
    ref = np.argmax(np.take_along_axis(nodes[:, None], rows[..., None].astype(np.int64), axis=2), axis=3)
    cand = ref.astype(np.int32)
    cand[:, 0, 1] = (ref[:, 0, 1] + 1) % V              # candidate 0 runs 1 token
    cand[:, 1, 2:] = -1                                 # candidate 1: 2 real tokens, then padding
    rows[:, 1, 2:] = -1
    cand[:, 2, 0] = (ref[:, 2, 0] + 1) % V              # candidate 2 runs 0 tokens
    t, a, best = oracle.greedy_tree(nodes, cand, rows)
    assert (a == 2).all() and (best == 1).all()
    np.testing.assert_array_equal(t[:, :2], cand[:, 1, :2])
    assert (t[:, 2:] == -1).all()                       # correction from the padded row, then padding


# ---------------------------------------------------------------------------
# Consistent top-k / top-p truncation of p and q (Ouroboros samples with
# top-p 0.8; the blog requires processors to be applied to target and draft
# alike)
# ---------------------------------------------------------------------------
def test_truncation_worked_examples():
    """Hand-worked cases of the definition (top-k keeps logits >= the k-th
    largest; top-p keeps a token when the kept mass strictly above it is below
    top_p of the kept mass)."""
    P = np.array([0.5, 0.3, 0.15, 0.05])
    z = np.log(P).astype(np.float32)
    cases = [
        (0, 0.8, [0.625, 0.375, 0, 0]),        # 0.5 < 0.8 keeps 0.3; 0.8 is not < 0.8
        (0, 0.81, [0.5 / 0.95, 0.3 / 0.95, 0.15 / 0.95, 0]),
        (0, 0.5, [1, 0, 0, 0]),                # 0.5 is not < 0.5
        (0, 0.49, [1, 0, 0, 0]),
        (2, 1.0, [0.625, 0.375, 0, 0]),
        (3, 1.0, [0.5 / 0.95, 0.3 / 0.95, 0.15 / 0.95, 0]),
        (3, 0.6, [0.625, 0.375, 0, 0]),        # top-p on the top-3 mass: 0.5/0.95 < 0.6
        (3, 0.5, [1, 0, 0, 0]),
        (4, 1.0, list(P)),
        (0, 1.0, list(P)),
    ]
    for top_k, top_p, want in cases:
        got, _ = oracle.truncated_row(z, 1.0, top_k, top_p)
        np.testing.assert_allclose(got, want, atol=2e-7, err_msg=f"top_k={top_k} top_p={top_p}")
    # ties at the boundary are kept together
    zt = np.array([1.0, 1.0, 0.0, 0.0], np.float32)
    got, _ = oracle.truncated_row(zt, 1.0, 1, 1.0)
    np.testing.assert_allclose(got, [0.5, 0.5, 0, 0], atol=1e-12)
    got, _ = oracle.truncated_row(zt, 1.0, 0, 0.3)
    np.testing.assert_allclose(got, [0.5, 0.5, 0, 0], atol=1e-12)
    # temperature applies before truncation: T = 0.5 squares and renormalises
    got, _ = oracle.truncated_row(z, 0.5, 0, 0.9)
    P2 = P ** 2 / (P ** 2).sum()               # [0.7042, 0.2535, 0.0634, 0.0070]
    np.testing.assert_allclose(got, [P2[0] / (P2[0] + P2[1]), P2[1] / (P2[0] + P2[1]), 0, 0], atol=1e-6)


def np_truncate(P, top_k, top_p):
    """Independent numpy statement of the truncation for probability rows."""
    out = np.zeros_like(P)
    for i, row in enumerate(P):
        keep = np.ones(len(row), bool)
        if 0 < top_k < len(row):
            keep &= row >= np.sort(row)[::-1][top_k - 1]
        if top_p < 1.0:
            M = row[keep].sum()
            above = np.array([row[keep & (row > v)].sum() for v in row])
            keep &= above < top_p * M
        out[i] = np.where(keep, row, 0.0) / row[keep].sum()
    return out


@pytest.mark.parametrize("top_k,top_p", [(3, 1.0), (0, 0.7), (5, 0.8)])
def test_v8_truncated_law(top_k, top_p):
    """With x drawn from the truncated draft q', every committed token follows
    the truncated target p' exactly (the rule's guarantee, applied to p', q')."""
    rng = np.random.default_rng(18)
    k = 3
    P = rng.dirichlet(np.ones(8), k + 1)
    Q = rng.dirichlet(np.ones(8), k)
    Pt, Qt = np_truncate(P, top_k, top_p), np_truncate(Q, top_k, top_p)
    pr = Probe(P, Q, 1.0, oracle.MUT_NONE)
    pr.run = lambda x, U: oracle.sample_truncated(
        np.broadcast_to(pr.z, (U.shape[0],) + pr.z.shape).copy(),
        np.broadcast_to(pr.y, (U.shape[0],) + pr.y.shape).copy(),
        np.broadcast_to(np.asarray(x, np.int32), (U.shape[0], k)).copy(),
        U.astype(np.float32), 1.0, top_k, top_p)
    safe = [int(np.argmax(np.minimum(Pt[i], Qt[i]) + 1e-3 * (Pt[i] > 0))) for i in range(k)]
    for i in range(k):
        law = np.zeros(8)
        for xv in range(8):
            if Qt[i, xv] == 0:
                continue
            x = safe.copy()
            x[i] = xv
            base = np.zeros(k + 1)
            a = pr.measure(x, base, i, lambda r: 1 if r is None else (r[1] > i))[0]
            law[xv] += Qt[i, xv] * a
            if a < 1.0:
                base[i] = a
                cdf = pr.measure(x, base, k, lambda r: 8 if r is None else (r[0][:, i] <= np.arange(8)))
                law += Qt[i, xv] * (1 - a) * np.diff(np.concatenate([[0.0], cdf]))
        np.testing.assert_allclose(law, Pt[i], atol=3e-6, err_msg=f"position {i}")


def test_top_k_one_is_greedy():
    rng = np.random.default_rng(19)
    n, k, V = 300, 4, 50
    z = rng.normal(0, 1, (n, k + 1, V)).astype(np.float32)
    y = (z[:, :k] + rng.normal(0, 1, (n, k, V))).astype(np.float32)
    x = np.argmax(y, axis=2).astype(np.int32)          # the truncated draft's only token
    u = u24(rng, (n, k + 1))
    ts, ns = oracle.sample_truncated(z, y, x, u, 1.0, top_k=1)
    tg, ng = oracle.greedy(z, x)
    np.testing.assert_array_equal(ns, ng)
    np.testing.assert_array_equal(ts, tg)


def test_truncation_off_is_the_rule():
    rng = np.random.default_rng(20)
    n, k, V = 200, 5, 40
    z = rng.normal(0, 2, (n, k + 1, V)).astype(np.float32)
    y = (z[:, :k] + rng.normal(0, 1, (n, k, V))).astype(np.float32)
    x = rng.integers(0, V, (n, k)).astype(np.int32)
    u = u24(rng, (n, k + 1))
    t1, n1 = oracle.sample(z, y, x, u, 0.8)
    for top_k, top_p in ((0, 1.0), (V, 1.0), (V + 5, 2.0)):
        t2, n2 = oracle.sample_truncated(z, y, x, u, 0.8, top_k, top_p)
        np.testing.assert_array_equal(t1, t2)
        np.testing.assert_array_equal(n1, n2)


# ---------------------------------------------------------------------------
# The exported probabilities and the draw's CDF intervals (used by the parity
# checks), pinned outside the functions themselves
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [0.7, 1.0, 1.3])
def test_token_probs_are_softmax_entries(T):
    """p_i(x_i), q_i(x_i) are softmax(z_i / T)[x_i] and softmax(y_i / T)[x_i]
    (scipy's softmax); an invalid token reports 0 for both."""
    import scipy.special
    rng = np.random.default_rng(31)
    k, V = 5, 257
    z = rng.normal(0, 2, (k + 1, V)).astype(np.float32)
    y = (z[:k] + rng.normal(0, 1, (k, V))).astype(np.float32)
    x = rng.integers(0, V, k).astype(np.int32)
    x[3] = V + 4                                   # outside the vocabulary
    px, qx = oracle.token_probs(z, y, x, T)
    for i in range(k):
        if i == 3:
            assert px[i] == 0.0 and qx[i] == 0.0
            continue
        ref_p = scipy.special.softmax(z[i].astype(np.float64) / T)[x[i]]
        ref_q = scipy.special.softmax(y[i].astype(np.float64) / T)[x[i]]
        np.testing.assert_allclose(px[i], ref_p, rtol=1e-12)
        np.testing.assert_allclose(qx[i], ref_q, rtol=1e-12)


def test_draw_intervals_tile_and_match_the_draws():
    """The intervals of all tokens tile [0, 1) in index order (zero-weight
    tokens get empty ones), and a uniform at an interval's midpoint makes the
    rule's own draw (pinned by the V = 8 law) pick that token: after a forced
    rejection (residual against the draft row) and for the bonus (target row)."""
    rng = np.random.default_rng(32)
    V, T = 8, 1.0
    P = rng.dirichlet(np.ones(V))
    P[2] = 0.0
    P /= P.sum()
    Q = rng.dirichlet(np.ones(V))
    with np.errstate(divide="ignore"):         # token 2 has p = 0: logit -inf
        z = np.log(np.stack([P, rng.dirichlet(np.ones(V))])).astype(np.float32)   # rows 0 and 1 (bonus)
    y = np.log(Q)[None].astype(np.float32)
    x0 = int(np.argmax(Q / np.maximum(P, 1e-30)))  # a token with q > p: rejectable
    for row, drow in ((0, y[0]), (1, None)):
        iv = [oracle.draw_interval(z[row], drow, T, t) for t in range(V)]
        lo = np.array([a for a, _, _ in iv])
        hi = np.array([b for _, b, _ in iv])
        w = np.array([c for _, _, c in iv])
        assert lo[0] == 0.0 and abs(hi[-1] - 1.0) < 1e-12
        np.testing.assert_allclose(lo[1:], hi[:-1], atol=1e-15)
        assert ((hi - lo > 0) == (w > 0)).all()
        for t in range(V):
            if w[t] <= 0:
                continue
            um = np.float32((lo[t] + hi[t]) / 2)
            if row == 0:       # reject x0 (u0 just below 1), then draw with um
                u = np.array([[np.float32(1 - 2 ** -24), um]], np.float32)
            else:              # accept x0 (u0 = 0 and p(x0) > 0 needed), bonus with um
                u = np.array([[0.0, um]], np.float32)
            xs = np.array([[x0 if row == 0 else int(np.argmax(P))]], np.int32)
            toks, na = oracle.sample(z[None], y[None], xs, u, T)
            assert na[0] == (0 if row == 0 else 1)
            assert toks[0, na[0]] == t, (row, t, toks)


def test_probability_error_floor():
    """The exported probabilities are float32: relative error above float32's
    smallest normal number, absolute (against that number) below it."""
    from oracle.parity import FP32_MIN_NORMAL, prob_error
    assert prob_error(np.float32(0.5), 0.5) == 0.0
    assert abs(prob_error(np.float32(1.0 + 2 ** -20), 1.0) - 2 ** -20) < 1e-12
    # a true value deep below the float32 range, exported as 0: error = value / 2^-126
    assert prob_error(np.float32(0.0), 1e-60) < 1e-20
    # a denormal exported one unit off is still tiny against the floor
    assert prob_error(np.float32(2 ** -140), 2 ** -140 + 2 ** -149) < 2 ** -22
    # a normal value off by 1e-4 relative stays 1e-4
    assert abs(prob_error(np.float32(1e-10 * (1 + 1e-4)), 1e-10) - 1e-4) < 1e-6
    assert FP32_MIN_NORMAL == 2.0 ** -126
