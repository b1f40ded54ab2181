"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Greedy and candidate selection: bit-exact.  Sampling: exact except in rounds
where the oracle's own decision lies within 1e-5 of its boundary (counted, and
checked for validity: see oracle/parity.py); exported p_i(x_i), q_i(x_i)
within 1e-5 relative.  Shapes span several workgroup slices and a ragged tail
(V not a multiple of 8, rows not 16-byte aligned, V < 8, k = 1 and 63), the
five workloads at full size, and the degenerate cases of the rule.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from oracle import parity

pytestmark = pytest.mark.gpu

EPS = 1e-5
PROB_RTOL = 1e-5
DEV = "cuda"


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    import draft_verification_verify_amd as m
    return m


def f32(t):
    return t.float().cpu().numpy()


def npi(t):
    return t.cpu().numpy()


def corrupt_after_argmax(target, k, gen, p_keep=0.7):
    """Drafts equal to the target argmax for a random prefix, then random:
    greedy acceptance lengths spread over 0..k."""
    B, _, V = target.shape
    am = torch.argmax(target[:, :k].float(), dim=2).to(torch.int32)
    keep = torch.rand((B, k), generator=gen, device=target.device) < p_keep
    rnd = torch.randint(0, V, (B, k), generator=gen, device=target.device, dtype=torch.int32)
    return torch.where(keep, am, rnd)


def with_layout(t, layout, gen):
    """Return a view of `t` with the requested memory layout: 'dense', 'padded'
    (row stride V+1: not 16-byte aligned), or 'offset' (base shifted by one
    element inside a wider buffer)."""
    if layout == "dense":
        return t
    *lead, V = t.shape
    pad = 1 if layout == "padded" else 9
    big = torch.randn((*lead, V + pad), generator=gen, device=t.device).to(t.dtype)
    off = 0 if layout == "padded" else 1
    big[..., off:off + V] = t
    return big[..., off:off + V]


# ---------------------------------------------------------------------------
# greedy
# ---------------------------------------------------------------------------
SHAPES = [(1, 1, 1), (3, 2, 7), (5, 4, 8), (4, 3, 1000), (2, 5, 4097), (6, 4, 32000),
          (2, 63, 300), (1, 4, 128256), (9, 8, 12345)]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("B,k,V", SHAPES)
@pytest.mark.parametrize("layout", ["dense", "padded", "offset"])
def test_greedy_parity(sv, dtype, B, k, V, layout):
    g = torch.Generator(device=DEV).manual_seed(B * 7919 + k * 31 + V)
    w = synthetic.chain(B, k, V, dtype, seed=B + k + V, device=DEV)
    x = corrupt_after_argmax(w.target, k, g)
    tgt = with_layout(w.target, layout, g)
    toks, na = sv.greedy(tgt, x)
    torch.cuda.synchronize()
    bad, ot, on = parity.check_greedy(f32(w.target), npi(x), npi(toks), npi(na))
    assert not bad, (bad[:5], npi(toks)[bad[:3]], ot[bad[:3]])


def test_greedy_ties_zeros_and_masked_rows(sv):
    """Tie-heavy integer logits, -0.0/+0.0 ties, rows that are all -inf."""
    g = torch.Generator(device=DEV).manual_seed(5)
    B, k, V = 64, 6, 3001
    for dtype in (torch.float32, torch.float16, torch.bfloat16):
        z = torch.randint(-3, 3, (B, k + 1, V), generator=g, device=DEV).to(dtype)
        zero = z == 0
        neg = torch.rand(z.shape, generator=g, device=DEV) < 0.5
        z = torch.where(zero & neg, torch.tensor(-0.0, dtype=dtype, device=DEV), z)
        z[::7] = -float("inf")
        z[3, 2, :] = 2.0                  # a whole row tied: index 0
        x = corrupt_after_argmax(z, k, g, 0.8)
        toks, na = sv.greedy(z, x)
        torch.cuda.synchronize()
        bad, _, _ = parity.check_greedy(f32(z), npi(x), npi(toks), npi(na))
        assert not bad, (dtype, bad[:5])


def test_greedy_invalid_tokens(sv):
    g = torch.Generator(device=DEV).manual_seed(6)
    w = synthetic.chain(32, 5, 2000, "bf16", seed=6, device=DEV)
    x = corrupt_after_argmax(w.target, 5, g, 1.0)
    pos = torch.randint(0, 5, (32,), generator=g, device=DEV)
    bad_vals = torch.tensor([-1, 2000, 2001, -(2 ** 31), 2 ** 31 - 1], device=DEV, dtype=torch.int32)
    x[torch.arange(32, device=DEV), pos] = bad_vals[torch.arange(32, device=DEV) % 5]
    toks, na = sv.greedy(w.target, x)
    torch.cuda.synchronize()
    assert (npi(na) == npi(pos)).all()
    bad, _, _ = parity.check_greedy(f32(w.target), npi(x), npi(toks), npi(na))
    assert not bad


# ---------------------------------------------------------------------------
# sampling
# ---------------------------------------------------------------------------
def run_sample(sv, w, layout="dense", gen=None):
    tgt = with_layout(w.target, layout, gen) if layout != "dense" else w.target
    dft = with_layout(w.draft, layout, gen) if layout != "dense" else w.draft
    toks, na, px, qx = sv.sample(tgt, dft, w.tokens, w.uniforms, w.T, return_probs=True)
    torch.cuda.synchronize()
    return npi(toks), npi(na), npi(px), npi(qx)


def assert_sample_parity(w, toks, na, px, qx):
    z, y = f32(w.target), f32(w.draft)
    x, u = npi(w.tokens), npi(w.uniforms)
    rep = parity.check_sample(z, y, x, u, w.T, toks, na, eps=EPS)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    print(rep.summary())
    worst = parity.check_probs(z, y, x, w.T, px, qx)
    assert worst <= PROB_RTOL, worst
    return rep


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("B,k,V", SHAPES)
@pytest.mark.parametrize("T", [0.6, 1.0])
def test_sample_parity(sv, dtype, B, k, V, T):
    w = synthetic.chain(B, k, V, dtype, var_target=2.0, var_noise=0.5, T=T, seed=B * 3 + k + V,
                        device=DEV)
    toks, na, px, qx = run_sample(sv, w)
    assert_sample_parity(w, toks, na, px, qx)


@pytest.mark.parametrize("dtype,var_target,T", [
    ("fp32", 400.0, 0.1),      # LLM-sized logits (sd 20) at a low temperature: |m c| ~ 900
    ("bf16", 400.0, 0.1),
    ("fp16", 400.0, 0.3),
    ("fp32", 2.0, 25.0),       # a high temperature: near-uniform p and q
    ("bf16", 1e4, 1.0),        # logits of order 100-400
])
def test_sample_parity_extreme_scales(sv, dtype, var_target, T):
    """Large logits and low temperatures make z * c large; the acceptance
    ratios, draws and exported p(x), q(x) must still meet the same bar."""
    w = synthetic.chain(32, 6, 5003, dtype, var_target=var_target, var_noise=0.05 * var_target,
                        T=T, seed=int(var_target) + 7, device=DEV)
    toks, na, px, qx = run_sample(sv, w)
    assert_sample_parity(w, toks, na, px, qx)


@pytest.mark.parametrize("layout", ["padded", "offset"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_sample_parity_unaligned(sv, dtype, layout):
    g = torch.Generator(device=DEV).manual_seed(9)
    w = synthetic.chain(12, 4, 5003, dtype, var_noise=0.5, T=0.8, seed=17, device=DEV)
    toks, na, px, qx = run_sample(sv, w, layout, g)
    assert_sample_parity(w, toks, na, px, qx)


def test_sample_identical_draft_takes_bonus(sv):
    """p = q: every draft is accepted and the bonus is drawn from p_k."""
    w = synthetic.chain(64, 7, 3000, "bf16", T=1.3, seed=21, device=DEV)
    w.draft.copy_(w.target[:, :7])
    toks, na, px, qx = run_sample(sv, w)
    assert (na == 7).all()
    assert_sample_parity(w, toks, na, px, qx)


def test_sample_masked_tokens(sv):
    """Grammar-style masking: the same columns are -inf in target and draft."""
    g = torch.Generator(device=DEV).manual_seed(22)
    w = synthetic.chain(48, 5, 4000, "fp16", var_noise=1.0, T=1.0, seed=22, device=DEV)
    mask = torch.rand((48, 1, 4000), generator=g, device=DEV) < 0.4
    w.target.masked_fill_(mask, -float("inf"))
    w.draft.masked_fill_(mask, -float("inf"))
    w.tokens.copy_(synthetic.gumbel_max_sample(w.draft.reshape(-1, 4000), 1.0, g).reshape(48, 5))
    toks, na, px, qx = run_sample(sv, w)
    assert_sample_parity(w, toks, na, px, qx)
    m = npi(mask[:, 0])
    for b in range(48):
        assert not m[b, toks[b, : na[b] + 1]].any()


def test_sample_invalid_tokens(sv):
    g = torch.Generator(device=DEV).manual_seed(23)
    w = synthetic.chain(40, 6, 1000, "bf16", seed=23, device=DEV)
    w.draft.copy_(w.target[:, :6])                       # valid drafts always accepted
    pos = torch.randint(0, 6, (40,), generator=g, device=DEV)
    vals = torch.tensor([-1, 1000, 5000, -(2 ** 31)], device=DEV, dtype=torch.int32)
    w.tokens[torch.arange(40, device=DEV), pos] = vals[torch.arange(40, device=DEV) % 4]
    toks, na, px, qx = run_sample(sv, w)
    assert (na == npi(pos)).all()
    assert_sample_parity(w, toks, na, px, qx)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("u", [0.0, 1.0 - 2.0 ** -24])
def test_sample_extreme_uniforms(sv, dtype, u):
    """Uniforms at the ends of [0, 1): u = 0 accepts every draft of positive
    probability and draws the first token of positive weight; the largest
    float below 1 accepts only where p >= q (up to the counted tie band) and
    draws from the end of the CDF."""
    w = synthetic.chain(64, 6, 5000, dtype, var_noise=2.0, T=0.9, seed=31, device=DEV)
    w.uniforms.fill_(u)
    toks, na, px, qx = run_sample(sv, w)
    rep = assert_sample_parity(w, toks, na, px, qx)
    if u == 0.0:
        assert (na == 6).all()
    assert rep.rounds == 64


def test_sample_low_temperature_matches_greedy(sv):
    """Low temperature: the sampling path reproduces the greedy path's tokens
    (the greedy collapse), both through the library."""
    g = torch.Generator(device=DEV).manual_seed(24)
    B, k, V = 64, 5, 2048
    z = torch.randint(-20, 20, (B, k + 1, V), generator=g, device=DEV).float()
    am = torch.randint(0, V, (B, k + 1), generator=g, device=DEV)
    z.scatter_(2, am[..., None], 21.0)
    y = z[:, :k].clone()
    x = corrupt_after_argmax(z, k, g, 0.7)
    y.scatter_(2, x[..., None].long(), 40.0)           # the draft puts its mass on x
    u = (torch.rand((B, k + 1), generator=g, device=DEV) * 0.998 + 0.001).float()
    ts, ns = sv.sample(z, y, x, u, 0.02)
    tg, ng = sv.greedy(z, x)
    torch.cuda.synchronize()
    assert (npi(ns) == npi(ng)).all() and (npi(ts) == npi(tg)).all()


# ---------------------------------------------------------------------------
# candidates
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,C,L,R,V", [(1, 1, 1, 1, 5), (3, 2, 4, 4, 999), (5, 8, 8, 8, 3000),
                                       (4, 8, 8, 9, 3000), (2, 1, 63, 63, 500), (2, 1, 63, 64, 500),
                                       (6, 4, 16, 17, 20000)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_candidates_parity(sv, B, C, L, R, V, dtype):
    w = synthetic.candidates(B, C, L, R, V, dtype, spike=8.0, seed=B + C + L + V, device=DEV)
    toks, A, best = sv.greedy_candidates(w.target, w.tokens)
    torch.cuda.synchronize()
    bad, ot, oa, ob = parity.check_candidates(f32(w.target), npi(w.tokens), npi(toks), npi(A),
                                              npi(best))
    assert not bad, (bad[:5], npi(toks)[bad[:2]], ot[bad[:2]])


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
def test_workload1_rounds(sv):
    """B=1, k=4, V=32000 fp32: 1000 rounds, one call each, greedy and sampling."""
    w = synthetic.generate(1, device=DEV, B=1000)
    tg, ng, ts, ns = [], [], [], []
    for r in range(1000):
        a, b = sv.greedy(w.target[r:r + 1], w.tokens[r:r + 1])
        c, d = sv.sample(w.target[r:r + 1], w.draft[r:r + 1], w.tokens[r:r + 1],
                         w.uniforms[r:r + 1], w.T)
        tg.append(a); ng.append(b); ts.append(c); ns.append(d)
    torch.cuda.synchronize()
    tg, ng = npi(torch.cat(tg)), npi(torch.cat(ng))
    ts, ns = npi(torch.cat(ts)), npi(torch.cat(ns))
    z, y = f32(w.target), f32(w.draft)
    bad, _, _ = parity.check_greedy(z, npi(w.tokens), tg, ng)
    assert not bad
    rep = parity.check_sample(z, y, npi(w.tokens), npi(w.uniforms), w.T, ts, ns, eps=EPS)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    print("workload 1:", rep.summary())


def test_workload2(sv):
    """Sampling on three input sets; greedy on the same target logits as an
    extra check, with drafts that follow the argmax for a random prefix."""
    for s in range(3):
        w = synthetic.generate(2, device=DEV, set_index=s)
        toks, na, px, qx = run_sample(sv, w)
        rep = assert_sample_parity(w, toks, na, px, qx)
        print(f"workload 2 set {s}:", rep.summary())
        g = torch.Generator(device=DEV).manual_seed(200 + s)
        x = corrupt_after_argmax(w.target, w.tokens.shape[1], g, 0.8)
        gt, gn = sv.greedy(w.target, x)
        torch.cuda.synchronize()
        bad, _, _ = parity.check_greedy(f32(w.target), npi(x), npi(gt), npi(gn))
        assert not bad


@pytest.fixture(scope="module")
def w3():
    return synthetic.generate(3, device=DEV)


def test_workload3_sample(sv, w3):
    toks, na, px, qx = run_sample(sv, w3)
    rep = assert_sample_parity(w3, toks, na, px, qx)
    print("workload 3 sample:", rep.summary())


@pytest.mark.parametrize("drafts", ["argmax", "sampled"])
def test_workload3_greedy(sv, w3, drafts):
    """Greedy verification of workload 3 with greedy drafting (the draft's own
    argmax at each position, a draft model decoding at temperature 0) and
    with the sampled drafts."""
    x = synthetic.greedy_drafts(w3.draft) if drafts == "argmax" else w3.tokens
    toks, na = sv.greedy(w3.target, x)
    torch.cuda.synchronize()
    bad, _, on = parity.check_greedy(f32(w3.target), npi(x), npi(toks), npi(na))
    assert not bad
    print(f"workload 3 greedy, {drafts} drafts: mean committed", on.mean() + 1)


def test_workload3_deterministic(sv, w3):
    a = run_sample(sv, w3)
    b = run_sample(sv, w3)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    g1 = [npi(t) for t in sv.greedy(w3.target, w3.tokens)]
    g2 = [npi(t) for t in sv.greedy(w3.target, w3.tokens)]
    assert all(np.array_equal(u, v) for u, v in zip(g1, g2))


@pytest.mark.parametrize("cid", [1, 2, 4, 5])
def test_workloads_deterministic(sv, cid, request):
    """Every workload's entry points called twice on the same stream give
    bit-identical outputs (no floating-point atomics, fixed reduction
    order)."""
    w = request.getfixturevalue("w5") if cid == 5 else synthetic.generate(cid, device=DEV)
    if cid == 4:
        calls = [lambda: sv.greedy_candidates(w.target, w.tokens)]
    else:
        calls = [lambda: sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, return_probs=True),
                 lambda: sv.greedy(w.target, w.tokens)]
    for f in calls:
        a = [npi(t) for t in f()]
        b = [npi(t) for t in f()]
        assert all(np.array_equal(u, v) for u, v in zip(a, b))


def test_workload4(sv):
    w = synthetic.generate(4, device=DEV)
    toks, A, best = sv.greedy_candidates(w.target, w.tokens)
    torch.cuda.synchronize()
    bad, ot, oa, ob = parity.check_candidates(f32(w.target), npi(w.tokens), npi(toks), npi(A),
                                              npi(best))
    assert not bad
    print("workload 4: mean accepted", oa.mean())


@pytest.fixture(scope="module")
def w5():
    return synthetic.generate(5, device=DEV)


def check_sample_all(w, toks, na, chunk=64, probs_every=8, px=None, qx=None):
    """Every sequence of a large batch against the oracle, `chunk` sequences
    at a time (host copies stay near 1 GB); the exported p(x), q(x) on every
    `probs_every`-th sequence."""
    B = w.target.shape[0]
    x, u = npi(w.tokens), npi(w.uniforms)
    rep = parity.SampleReport()
    worst = 0.0
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        z, y = f32(w.target[b0:b1]), f32(w.draft[b0:b1])
        parity.check_sample(z, y, x[b0:b1], u[b0:b1], w.T, toks[b0:b1], na[b0:b1], eps=EPS,
                            report=rep, seq_ids=np.arange(b0, b1))
        if px is not None:
            sel = np.arange(b0, b1)
            sel = sel[sel % probs_every == 0] - b0
            worst = max(worst, parity.check_probs(z[sel], y[sel], x[b0:b1][sel], w.T, px[b0:b1][sel],
                                                  qx[b0:b1][sel]))
    return rep, worst


def check_greedy_all(w, x, toks, na, chunk=64):
    """Every sequence of a large batch, bit-exact; returns the mismatching ids."""
    B = w.target.shape[0]
    bad = []
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        bb, _, _ = parity.check_greedy(f32(w.target[b0:b1]), x[b0:b1], toks[b0:b1], na[b0:b1])
        bad += [b0 + i for i in bb]
    return bad


def test_workload5_sample(sv, w5):
    """Full B=512, k=16, V=128256 bf16 call: every sequence checked for the
    rule's invariants and against the oracle; p(x), q(x) on every 8th."""
    toks, na, px, qx = run_sample(sv, w5)
    x = npi(w5.tokens)
    assert ((na >= 0) & (na <= 16)).all()
    for b in range(512):
        assert (toks[b, : na[b]] == x[b, : na[b]]).all()
        assert 0 <= toks[b, na[b]] < 128256
        assert (toks[b, na[b] + 1:] == -1).all()
    rep, worst = check_sample_all(w5, toks, na, px=px, qx=qx)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    assert rep.rounds == 512
    assert worst <= PROB_RTOL, worst
    print("workload 5 sample:", rep.summary())


def test_workload5_vocabulary_shard(sv):
    """Workload 5 as one of 8 vocabulary shards (V = 16032 per row, the shape
    bench.py --vocab-shard 8 times): every sequence against the oracle,
    sampling and greedy."""
    w = synthetic.generate(5, device=DEV, V=16032)
    toks, na, px, qx = run_sample(sv, w)
    rep, worst = check_sample_all(w, toks, na, px=px, qx=qx, probs_every=2)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    assert rep.rounds == 512
    assert worst <= PROB_RTOL, worst
    gt, gn = sv.greedy(w.target, w.tokens)
    torch.cuda.synchronize()
    assert not check_greedy_all(w, npi(w.tokens), npi(gt), npi(gn))
    print("workload 5, one of 8 vocabulary shards:", rep.summary())


def test_workload5_greedy(sv, w5):
    """Every sequence, bit-exact, with the sampled drafts and with drafts that
    follow the argmax for a random prefix (longer accepted runs)."""
    g = torch.Generator(device=DEV).manual_seed(505)
    for x in (w5.tokens, corrupt_after_argmax(w5.target, 16, g, 0.85)):
        toks, na = sv.greedy(w5.target, x)
        torch.cuda.synchronize()
        assert not check_greedy_all(w5, npi(x), npi(toks), npi(na))


# ---------------------------------------------------------------------------
# verification by-products (Ouroboros 3.4.4, Eq. 10) and lenience (Cascade)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("B,k,V", [(1, 1, 1), (5, 4, 1000), (9, 8, 12345), (3, 63, 300), (2, 16, 128256)])
def test_greedy_ext_parity(sv, dtype, B, k, V):
    g = torch.Generator(device=DEV).manual_seed(B + k + V)
    w = synthetic.chain(B, k, V, dtype, seed=B * 5 + k + V, device=DEV)
    x = corrupt_after_argmax(w.target, k, g, 0.8)
    toks, na, v, mask, cnt = sv.greedy_ext(w.target, x)
    t2, n2 = sv.greedy(w.target, x)
    torch.cuda.synchronize()
    assert np.array_equal(npi(toks), npi(t2)) and np.array_equal(npi(na), npi(n2))
    z = f32(w.target)
    bad, _, _ = parity.check_greedy(z, npi(x), npi(toks), npi(na))
    assert not bad
    bad = parity.check_greedy_matches(z, npi(x), npi(v), npi(mask), npi(cnt))
    assert not bad, bad[:5]
    assert (npi(cnt) >= npi(na)).all()


def test_greedy_ext_workload3(sv, w3):
    """The #Match by-products on workload 3 with greedy drafting."""
    x = synthetic.greedy_drafts(w3.draft)
    toks, na, v, mask, cnt = sv.greedy_ext(w3.target, x)
    torch.cuda.synchronize()
    z = f32(w3.target)
    assert not parity.check_greedy(z, npi(x), npi(toks), npi(na))[0]
    assert not parity.check_greedy_matches(z, npi(x), npi(v), npi(mask), npi(cnt))
    print("workload 3 greedy: mean #Match", npi(cnt).mean(), "mean accepted", npi(na).mean())


@pytest.mark.parametrize("B,C,L,R,V", [(3, 2, 4, 4, 999), (4, 8, 8, 9, 3000), (2, 1, 63, 64, 500)])
def test_candidates_ext_parity(sv, B, C, L, R, V):
    w = synthetic.candidates(B, C, L, R, V, "bf16", seed=B + C + L + V + 1, device=DEV)
    toks, A, best, v = sv.greedy_candidates_ext(w.target, w.tokens)
    torch.cuda.synchronize()
    z = f32(w.target)
    bad, _, _, _ = parity.check_candidates(z, npi(w.tokens), npi(toks), npi(A), npi(best))
    assert not bad
    assert not parity.check_row_argmax(z, npi(v))


def test_candidates_ext_workload4(sv):
    w = synthetic.generate(4, device=DEV)
    toks, A, best, v = sv.greedy_candidates_ext(w.target, w.tokens)
    torch.cuda.synchronize()
    z = f32(w.target)
    assert not parity.check_candidates(z, npi(w.tokens), npi(toks), npi(A), npi(best))[0]
    assert not parity.check_row_argmax(z, npi(v))


def test_lenience_one_is_bitwise_the_rule(sv, w3):
    a = sv.sample(w3.target, w3.draft, w3.tokens, w3.uniforms, w3.T, return_probs=True)
    b = sv.sample_lenient(w3.target, w3.draft, w3.tokens, w3.uniforms, w3.T, 1.0, return_probs=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert np.array_equal(npi(u), npi(v))


@pytest.mark.parametrize("lenience", [1.5, 3.0, 1e6])
@pytest.mark.parametrize("dtype,B,k,V", [("bf16", 32, 6, 5003), ("fp16", 8, 4, 32000), ("fp32", 16, 8, 999)])
def test_lenient_parity(sv, lenience, dtype, B, k, V):
    w = synthetic.chain(B, k, V, dtype, var_noise=1.5, T=0.9, seed=B + k + V, device=DEV)
    toks, na, px, qx = sv.sample_lenient(w.target, w.draft, w.tokens, w.uniforms, w.T, lenience,
                                         return_probs=True)
    torch.cuda.synchronize()
    z, y = f32(w.target), f32(w.draft)
    rep = parity.check_sample(z, y, npi(w.tokens), npi(w.uniforms), w.T, npi(toks), npi(na),
                              eps=EPS, lenience=lenience)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    assert parity.check_probs(z, y, npi(w.tokens), w.T, npi(px), npi(qx)) <= PROB_RTOL
    print(f"lenience {lenience}:", rep.summary())


# ---------------------------------------------------------------------------
# token tree (Ouroboros Figure 3: each node scored once)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,N,C,L,R,V", [(1, 1, 1, 1, 1, 5), (7, 10, 4, 5, 5, 999), (5, 20, 8, 8, 9, 3001),
                                         (3, 70, 1, 63, 64, 300), (4, 43, 8, 8, 8, 20000)])
def test_tree_parity(sv, B, N, C, L, R, V):
    g = torch.Generator(device=DEV).manual_seed(B * N + C + L + V)
    nodes = (torch.randn((B, N, V), generator=g, device=DEV) * 2).to(torch.bfloat16)
    rows = torch.randint(0, N, (B, C, R), generator=g, device=DEV, dtype=torch.int32)
    if N > 2:                                    # a few invalid row indices
        rows[0, 0, -1] = N
        rows[-1, C - 1, 0] = -7
    ref = torch.gather(torch.argmax(nodes.float(), dim=2), 1, rows.clamp(0, N - 1).long().reshape(B, -1))
    ref = ref.reshape(B, C, R)[:, :, :L].to(torch.int32)
    keep = torch.rand((B, C, L), generator=g, device=DEV) < 0.85
    cand = torch.where(keep, ref, torch.randint(0, V, (B, C, L), generator=g, device=DEV, dtype=torch.int32))
    toks, A, best = sv.greedy_tree(nodes, cand, rows)
    torch.cuda.synchronize()
    ot, oa, ob = oracle.greedy_tree(f32(nodes), npi(cand), npi(rows))
    assert np.array_equal(ot, npi(toks)) and np.array_equal(oa, npi(A)) and np.array_equal(ob, npi(best))


def test_tree_padding_slots(sv):
    """Short candidates padded with token -1 at row -1 (a tree builder's
    padding): the padded positions never match, so no -1 is ever committed
    as an accepted token, and the GPU equals the oracle."""
    B, N, C, L, V = 24, 9, 4, 6, 3001
    g = torch.Generator(device=DEV).manual_seed(2024)
    nodes = (torch.randn((B, N, V), generator=g, device=DEV) * 2).to(torch.bfloat16)
    rows = torch.randint(0, N, (B, C, L), generator=g, device=DEV, dtype=torch.int32)
    ref = torch.gather(torch.argmax(nodes.float(), dim=2), 1, rows.long().reshape(B, -1)).reshape(B, C, L)
    cand = ref.to(torch.int32)
    lens = torch.randint(0, L + 1, (B, C), generator=g, device=DEV)
    pad = torch.arange(L, device=DEV)[None, None, :] >= lens[:, :, None]
    cand[pad] = -1
    rows[pad] = -1
    toks, A, best = sv.greedy_tree(nodes, cand, rows)
    torch.cuda.synchronize()
    ot, oa, ob = oracle.greedy_tree(f32(nodes), npi(cand), npi(rows))
    assert np.array_equal(ot, npi(toks)) and np.array_equal(oa, npi(A)) and np.array_equal(ob, npi(best))
    assert np.array_equal(npi(A), npi(lens).max(axis=1))
    t, a = npi(toks), npi(A)
    for b in range(B):
        assert (t[b, :a[b]] >= 0).all()


def test_tree_workload4_equals_flat(sv):
    w = synthetic.generate(4, device=DEV)
    nodes, rows = synthetic.as_tree(w)
    assert nodes.shape[1] == 43
    t1, a1, b1 = sv.greedy_tree(nodes, w.tokens, rows)
    t2, a2, b2 = sv.greedy_candidates(w.target, w.tokens)
    torch.cuda.synchronize()
    for u, v in ((t1, t2), (a1, a2), (b1, b2)):
        assert np.array_equal(npi(u), npi(v))
    ot, oa, ob = oracle.greedy_tree(f32(nodes), npi(w.tokens), npi(rows))
    assert np.array_equal(ot, npi(t1)) and np.array_equal(oa, npi(a1)) and np.array_equal(ob, npi(b1))


# ---------------------------------------------------------------------------
# early exit: the same results, bit for bit, from fewer rows
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("B,k,V", [(1, 1, 1), (5, 4, 1000), (9, 8, 12345), (3, 63, 300), (6, 16, 32000),
                                   (2, 3, 100003),    # 24 slices per row, merged in three batches
                                   (129, 8, 9001)])   # 2193 short rows, one slice each
@pytest.mark.parametrize("noise", [0.3, 3.0])
def test_lazy_equals_full(sv, dtype, B, k, V, noise):
    w = synthetic.chain(B, k, V, dtype, var_noise=noise, T=0.8, seed=B * 11 + k + V, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(B + k)
    x = corrupt_after_argmax(w.target, k, g, 0.9)
    a = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T)
    b = sv.sample_lazy(w.target, w.draft, w.tokens, w.uniforms, w.T)
    c = sv.greedy(w.target, x)
    d = sv.greedy_lazy(w.target, x)
    torch.cuda.synchronize()
    for u, v in zip(a + c, b + d):
        assert np.array_equal(npi(u), npi(v))
    bad, _, _ = parity.check_greedy(f32(w.target), npi(x), npi(d[0]), npi(d[1]))
    assert not bad
    rep = parity.check_sample(f32(w.target), f32(w.draft), npi(w.tokens), npi(w.uniforms), w.T,
                              npi(b[0]), npi(b[1]), eps=EPS)
    assert rep.ok(), (rep.summary(), rep.failures[:3])


def test_lazy_full_acceptance_and_masking(sv):
    """Every draft accepted (p = q): every window runs and the bonus is drawn;
    invalid tokens stop a sequence mid-window."""
    w = synthetic.chain(40, 20, 3000, "bf16", T=1.1, seed=41, device=DEV)
    w.draft.copy_(w.target[:, :20])
    w.tokens[5, 7] = -3
    w.tokens[9, 13] = 3000
    a = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T)
    b = sv.sample_lazy(w.target, w.draft, w.tokens, w.uniforms, w.T)
    torch.cuda.synchronize()
    assert np.array_equal(npi(a[0]), npi(b[0])) and np.array_equal(npi(a[1]), npi(b[1]))
    na = npi(b[1])
    assert na[5] == 7 and na[9] == 13 and (np.delete(na, [5, 9]) == 20).all()


@pytest.mark.parametrize("cid", [3, 5])
def test_lazy_workloads(sv, cid):
    w = synthetic.generate(cid, device=DEV)
    a = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T)
    b = sv.sample_lazy(w.target, w.draft, w.tokens, w.uniforms, w.T)
    c = sv.greedy(w.target, w.tokens)
    d = sv.greedy_lazy(w.target, w.tokens)
    torch.cuda.synchronize()
    for u, v in zip(a + c, b + d):
        assert np.array_equal(npi(u), npi(v))


# ---------------------------------------------------------------------------
# streams and the measurement variants
# ---------------------------------------------------------------------------
def test_side_stream_and_timed_variants(sv):
    """Calls on a side stream equal calls on the current one; with a pair of
    the caller's events every entry point family records them around its
    streaming kernel (a positive duration) and computes the same result."""
    w = synthetic.chain(16, 4, 20000, "bf16", seed=31, device=DEV)
    ref = run_sample(sv, w)
    ref_g = [npi(t) for t in sv.greedy_ext(w.target, w.tokens)]
    c = synthetic.candidates(4, 3, 5, 5, 7001, "bf16", seed=9, device=DEV)
    ref_c = [npi(t) for t in sv.greedy_candidates_ext(c.target, c.tokens)]
    nodes, rows = synthetic.as_tree(c)
    ref_t = [npi(t) for t in sv.greedy_tree(nodes, c.tokens, rows)]
    ref_tr = [npi(t) for t in sv.sample_truncated(w.target, w.draft, w.tokens, w.uniforms, w.T, 20, 0.9)]
    ref_l = [npi(t) for t in sv.sample_lenient(w.target, w.draft, w.tokens, w.uniforms, w.T, 2.0)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(9)]
    with torch.cuda.stream(s):
        out = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, return_probs=True, events=evs[0])
        got = [
            (ref_g[:2], sv.greedy(w.target, w.tokens, events=evs[1])),
            (ref_g, sv.greedy_ext(w.target, w.tokens, events=evs[2])),
            (ref_c[:3], sv.greedy_candidates(c.target, c.tokens, events=evs[3])),
            (ref_c, sv.greedy_candidates_ext(c.target, c.tokens, events=evs[4])),
            (ref_t, sv.greedy_tree(nodes, c.tokens, rows, events=evs[5])),
            (ref_tr, sv.sample_truncated(w.target, w.draft, w.tokens, w.uniforms, w.T, 20, 0.9,
                                         events=evs[6])),
            (ref_l, sv.sample_lenient(w.target, w.draft, w.tokens, w.uniforms, w.T, 2.0, events=evs[7])),
            (ref[:2], sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, events=evs[8])),
        ]
    torch.cuda.synchronize()
    for a, b in zip(ref, out):
        assert np.array_equal(a, npi(b))
    for want, have in got:
        for a, b in zip(want, have):
            assert np.array_equal(a, npi(b))
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    assert all(m > 0 for m in ms), ms


# ---------------------------------------------------------------------------
# extremes of the shape space
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("V", [262144, 262147])
def test_large_vocabulary(sv, V):
    """Vocabularies past the workloads' (262144 is the largest in common use):
    more slices per row and a ragged tail at the odd size."""
    g = torch.Generator(device=DEV).manual_seed(V)
    w = synthetic.chain(4, 3, V, "bf16", var_target=3.0, var_noise=2.0, spike=8.0, seed=V, device=DEV)
    rep = assert_sample_parity(w, *run_sample(sv, w))
    assert rep.rounds == 4
    x = corrupt_after_argmax(w.target, 3, g)
    toks, na = sv.greedy(w.target, x)
    torch.cuda.synchronize()
    bad, _, _ = parity.check_greedy(f32(w.target), npi(x), npi(toks), npi(na))
    assert not bad


# 1100 x 16 x 131072 target and 1100 x 15 x 131072 draft logits: both
# tensors hold more than 2^31 elements (4.6 and 4.3 GB in bf16). Target rows
# of sequences 1024.. and draft rows of sequences 1093.. start past element
# 2^31, so a 32-bit element offset anywhere in the path would read the wrong
# rows there.
HUGE = dict(B=1100, k=15, V=131072)
HUGE_IDX = np.array([0, 1, 700, 1023, 1024, 1092, 1093, 1099])


def huge_workload():
    w = synthetic.chain(HUGE["B"], HUGE["k"], HUGE["V"], "bf16", var_target=3.0, var_noise=1.0,
                        seed=2 ** 31, device=DEV)
    assert w.target.numel() > 2 ** 31 and w.draft.numel() > 2 ** 31
    return w


def test_tensors_past_2_31_elements(sv):
    """Sampling, greedy and early exit on logit tensors of more than 2^31
    elements; the sequences on either side of element 2^31 are checked
    against the oracle, early exit against the full pass on every sequence."""
    w, idx = huge_workload(), HUGE_IDX
    B, k = HUGE["B"], HUGE["k"]
    ti = torch.as_tensor(idx, device=DEV)
    toks, na, px, qx = run_sample(sv, w)
    x, u = npi(w.tokens), npi(w.uniforms)
    z, y = f32(w.target[ti]), f32(w.draft[ti])
    rep = parity.check_sample(z, y, x[idx], u[idx], w.T, toks[idx], na[idx], eps=EPS, seq_ids=idx)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    assert parity.check_probs(z, y, x[idx], w.T, px[idx], qx[idx]) <= PROB_RTOL
    lz = sv.sample_lazy(w.target, w.draft, w.tokens, w.uniforms, w.T)
    g = torch.Generator(device=DEV).manual_seed(B)
    xg = corrupt_after_argmax(w.target, k, g, 0.9)
    gt, gn = sv.greedy(w.target, xg)
    gl = sv.greedy_lazy(w.target, xg)
    torch.cuda.synchronize()
    assert np.array_equal(npi(lz[0]), toks) and np.array_equal(npi(lz[1]), na)
    assert np.array_equal(npi(gl[0]), npi(gt)) and np.array_equal(npi(gl[1]), npi(gn))
    bad, _, _ = parity.check_greedy(z, npi(xg)[idx], npi(gt)[idx], npi(gn)[idx])
    assert not bad
    print("past 2^31 elements:", rep.summary(), "greedy accepted", npi(gn)[idx])
    del w, lz, gt, gn, gl
    torch.cuda.empty_cache()


def test_many_short_rows(sv):
    """4096 sequences of 300-token rows: far more sequences than workgroups
    per sequence, one slice per row."""
    g = torch.Generator(device=DEV).manual_seed(4096)
    w = synthetic.chain(4096, 2, 300, "fp16", seed=4096, device=DEV)
    assert_sample_parity(w, *run_sample(sv, w))
    x = corrupt_after_argmax(w.target, 2, g)
    toks, na = sv.greedy(w.target, x)
    torch.cuda.synchronize()
    bad, _, _ = parity.check_greedy(f32(w.target), npi(x), npi(toks), npi(na))
    assert not bad


# ---------------------------------------------------------------------------
# a seeded sweep over random shapes, dtypes, temperatures, scales and layouts
# ---------------------------------------------------------------------------
def random_case(i):
    """Case i of the sweep: log-uniform V in [1, 70000] (ragged tails), k up
    to 63, temperatures 0.05-5, logit variances 0.5-100, three layouts; the
    oracle's work is capped at 6e6 elements per case."""
    r = np.random.default_rng(9000 + i)
    dtype = ["fp32", "fp16", "bf16"][int(r.integers(3))]
    k = int(r.choice([1, 2, 3, 5, 8, 16, 31, 63]))
    V = max(1, int(np.exp(r.uniform(0.0, np.log(70000.0)))))
    B = int(r.integers(1, 41))
    while B > 1 and B * (2 * k + 1) * V > 6_000_000:
        B //= 2
    V = min(V, max(1, 6_000_000 // (B * (2 * k + 1))))
    T = float(np.exp(r.uniform(np.log(0.05), np.log(5.0))))
    var_t = float(r.choice([0.5, 2.0, 9.0, 100.0]))
    layout = ["dense", "padded", "offset"][int(r.integers(3))]
    return dtype, B, k, V, T, var_t, layout


@pytest.mark.parametrize("i", range(24))
def test_random_cases(sv, i):
    dtype, B, k, V, T, var_t, layout = random_case(i)
    print(f"case {i}: {dtype} B={B} k={k} V={V} T={T:.3f} var={var_t} {layout}", flush=True)
    w = synthetic.chain(B, k, V, dtype, var_target=var_t, var_noise=0.3 * var_t, T=T, seed=7000 + i,
                        device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(i)
    toks, na, px, qx = run_sample(sv, w, layout, gen)
    assert_sample_parity(w, toks, na, px, qx)
    # the layout changes only how rows are loaded: the dense call agrees bit for
    # bit, and so does early exit
    a = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T)
    lz = sv.sample_lazy(w.target, w.draft, w.tokens, w.uniforms, w.T)
    torch.cuda.synchronize()
    assert np.array_equal(toks, npi(a[0])) and np.array_equal(na, npi(a[1]))
    assert np.array_equal(npi(lz[0]), npi(a[0])) and np.array_equal(npi(lz[1]), npi(a[1]))
    # greedy on drafts that follow the argmax for a while
    x = corrupt_after_argmax(w.target, k, gen)
    g = sv.greedy(with_layout(w.target, layout, gen), x)
    gl = sv.greedy_lazy(w.target, x)
    torch.cuda.synchronize()
    bad, _, _ = parity.check_greedy(f32(w.target), npi(x), npi(g[0]), npi(g[1]))
    assert not bad
    assert np.array_equal(npi(gl[0]), npi(g[0])) and np.array_equal(npi(gl[1]), npi(g[1]))
    # the lenient rule with a random l >= 1
    lenience = 1.0 + float(np.random.default_rng(i).exponential(2.0))
    lt, ln = sv.sample_lenient(w.target, w.draft, w.tokens, w.uniforms, w.T, lenience)
    torch.cuda.synchronize()
    rep = parity.check_sample(f32(w.target), f32(w.draft), npi(w.tokens), npi(w.uniforms), w.T,
                              npi(lt), npi(ln), eps=EPS, lenience=lenience)
    assert rep.ok(), (lenience, rep.summary(), rep.failures[:3])


def random_candidate_case(i):
    """Case i: C x L up to 64 scored tokens, R = L or L+1, log-uniform V in
    [1, 60000], all three dtypes; the oracle's work capped at 8e6 elements."""
    r = np.random.default_rng(8000 + i)
    dtype = ["fp32", "fp16", "bf16"][int(r.integers(3))]
    C = int(r.integers(1, 9))
    L = int(r.integers(1, min(63, 64 // C) + 1))
    R = L + int(r.integers(2))
    V = max(1, int(np.exp(r.uniform(0.0, np.log(60000.0)))))
    B = int(r.integers(1, 25))
    while B > 1 and B * C * R * V > 8_000_000:
        B //= 2
    V = min(V, max(1, 8_000_000 // (B * C * R)))
    return dtype, B, C, L, R, V


@pytest.mark.parametrize("i", range(16))
def test_random_candidate_cases(sv, i):
    dtype, B, C, L, R, V = random_candidate_case(i)
    print(f"case {i}: {dtype} B={B} C={C} L={L} R={R} V={V}", flush=True)
    w = synthetic.candidates(B, C, L, R, V, dtype, spike=8.0, seed=8000 + i, device=DEV)
    toks, A, best = sv.greedy_candidates(w.target, w.tokens)
    et, ea, eb, ev = sv.greedy_candidates_ext(w.target, w.tokens)
    # the same rows as a token tree: node rows in a shuffled order, mapped back
    g = torch.Generator(device=DEV).manual_seed(i)
    perm = torch.randperm(C * R, generator=g, device=DEV)
    nodes = w.target.reshape(B, C * R, V)[:, perm].contiguous()
    inv = torch.argsort(perm).to(torch.int32)
    rows = inv.reshape(1, C, R).expand(B, C, R).contiguous()
    tt, ta, tb = sv.greedy_tree(nodes, w.tokens, rows)
    torch.cuda.synchronize()
    bad, _, _, _ = parity.check_candidates(f32(w.target), npi(w.tokens), npi(toks), npi(A), npi(best))
    assert not bad, bad[:5]
    for u, v in ((et, toks), (ea, A), (eb, best), (tt, toks), (ta, A), (tb, best)):
        assert np.array_equal(npi(u), npi(v))
    assert not parity.check_row_argmax(f32(w.target).reshape(B * C * R, V), npi(ev).reshape(-1))
