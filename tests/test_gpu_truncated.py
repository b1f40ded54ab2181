"""Parity of truncated sampling verification (top-k, then top-p, on target and
draft rows alike) with the CPU oracle, on the GPU, through the C ABI.

Exact except in rounds the oracle marks as boundary cases: an acceptance or a
draw within 1e-5 of its threshold, or a row whose kept-mass fraction lies
within 1e-5 of top_p at the top-p boundary (the GPU's fixed-point masses may
then keep the neighbouring set); such rounds are counted and checked for
validity (oracle/parity.py).  Exported p'(x), q'(x) within 1e-5 relative.
The proposer's drafts are drawn from the truncated q' itself, as a serving
engine that applies the same processor to the draft would.
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


def truncated_drafts(y, T, top_k, top_p, seed):
    """Draft tokens drawn from q' = the truncated draft rows (the proposer's
    side of a consistent processor), one per row of y [B, k, V]."""
    rng = np.random.default_rng(seed)
    B, k, V = y.shape
    x = np.zeros((B, k), np.int32)
    for b in range(B):
        for i in range(k):
            q, _ = oracle.truncated_row(y[b, i], T, top_k, top_p)
            x[b, i] = rng.choice(V, p=q / q.sum())
    return x


def workload(B, k, V, dtype, seed, top_k, top_p, T=None):
    w = synthetic.chain(B, k, V, dtype, seed=seed, device=DEV)
    T = w.T if T is None else T
    y = f32(w.draft)
    x = truncated_drafts(y, T, top_k, top_p, seed)
    return w, T, torch.from_numpy(x).to(DEV)


def check(sv, w, T, x, top_k, top_p, tgt=None, dft=None):
    tgt = w.target if tgt is None else tgt
    dft = w.draft if dft is None else dft
    toks, na, px, qx = sv.sample_truncated(tgt, dft, x, w.uniforms, T, top_k, top_p,
                                           return_probs=True)
    torch.cuda.synchronize()
    z, y = f32(w.target), f32(w.draft)
    xx, u = npi(x), npi(w.uniforms)
    rep = parity.check_sample_truncated(z, y, xx, u, T, top_k, top_p, npi(toks), npi(na), eps=EPS)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    print(rep.summary())
    worst, skipped = parity.check_probs_truncated(z, y, xx, T, top_k, top_p, npi(px), npi(qx))
    assert worst <= PROB_RTOL, worst
    return rep, npi(toks), npi(na)


SETTINGS = [(50, 1.0), (0, 0.8), (50, 0.9), (5, 0.95), (0, 0.3), (1000, 0.99)]


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("top_k,top_p", SETTINGS)
def test_truncated_parity(sv, dtype, top_k, top_p):
    B, k, V = 24, 5, 32000
    w, T, x = workload(B, k, V, dtype, 11 + top_k, top_k, top_p)
    rep, _, _ = check(sv, w, T, x, top_k, top_p)
    assert rep.exact >= rep.rounds - 2


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("B,k,V", [(8, 3, 4097), (4, 8, 1000), (3, 2, 7), (2, 4, 9), (5, 1, 100)])
@pytest.mark.parametrize("top_k,top_p", [(3, 1.0), (0, 0.7), (4, 0.6)])
def test_truncated_ragged_shapes(sv, dtype, B, k, V, top_k, top_p):
    w, T, x = workload(B, k, V, dtype, B + k + V, top_k, top_p)
    check(sv, w, T, x, top_k, top_p)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("u", [0.0, 1.0 - 2.0 ** -24])
def test_truncated_extreme_uniforms(sv, dtype, u):
    """Uniforms at the ends of [0, 1) on truncated rows: u = 0 draws the
    lowest-index token of the kept set, the largest float below 1 the
    highest; every draw must avoid the truncated-away tokens."""
    w, T, x = workload(32, 4, 6000, dtype, 33, 50, 0.9)
    w.uniforms.fill_(u)
    rep, _, _ = check(sv, w, T, x, 50, 0.9)
    assert rep.rounds == 32


def test_truncated_many_rows_per_workgroup(sv):
    """More rows than workgroups, at a vocabulary whose last round of loads
    is partly past the row end (V = 152064): each workgroup streams several
    rows, target and draft rows in turn."""
    w, T, x = workload(64, 4, 152064, "fp16", 152, 50, 0.9)
    check(sv, w, T, x, 50, 0.9)


@pytest.mark.parametrize("top_k,top_p", [(50, 0.9), (0, 0.8)])
def test_truncated_16bit_equals_fp32_at_full_size(sv, top_k, top_p):
    """At the full 512 x 16 x 128256 bf16 size, every row: the same rows
    upcast to fp32 (exact) go through the fp32 kernels (top-k 50: the fp32
    candidate lists, 256 threads per row; top-p alone: the radix passes)
    instead of the 16-bit ones, and the two must agree bit for bit (same keep
    set, same fixed-point masses, so the same tokens and the same p'(x),
    q'(x))."""
    w = synthetic.generate(5, device=DEV)
    a = sv.sample_truncated(w.target, w.draft, w.tokens, w.uniforms, w.T, top_k, top_p,
                            return_probs=True)
    b = sv.sample_truncated(w.target.float(), w.draft.float(), w.tokens, w.uniforms, w.T, top_k,
                            top_p, return_probs=True)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)


@pytest.mark.parametrize("layout", ["padded", "offset"])
def test_truncated_unaligned_rows(sv, layout):
    """Rows that are not 16-byte aligned take the element-load path."""
    B, k, V = 12, 4, 5003
    w, T, x = workload(B, k, V, "fp16", 77, 40, 0.9)
    g = torch.Generator(device=DEV).manual_seed(3)

    def lay(t):
        *lead, V_ = t.shape
        pad = 1 if layout == "padded" else 9
        big = torch.randn((*lead, V_ + pad), generator=g, device=DEV).to(t.dtype)
        off = 0 if layout == "padded" else 1
        big[..., off:off + V_] = t
        return big[..., off:off + V_]

    check(sv, w, T, x, 40, 0.9, tgt=lay(w.target), dft=lay(w.draft))


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_truncated_ties_and_masked_tokens(sv, dtype):
    """Integer logits (large tie groups straddle the top-k and top-p
    boundaries, which keep or drop a group whole), -0.0 beside +0.0, and
    -inf (masked) tokens."""
    g = torch.Generator(device=DEV).manual_seed(21)
    B, k, V = 16, 4, 3001
    tdt = synthetic.DTYPES[dtype]
    z = torch.randint(-4, 4, (B, k + 1, V), generator=g, device=DEV).to(tdt)
    y = torch.randint(-4, 4, (B, k, V), generator=g, device=DEV).to(tdt)
    neg = torch.rand(z.shape, generator=g, device=DEV) < 0.5
    z = torch.where((z == 0) & neg, torch.tensor(-0.0, dtype=tdt, device=DEV), z)
    mask = torch.rand(z.shape, generator=g, device=DEV) < 0.2
    z = z.masked_fill(mask, -float("inf"))
    y = y.masked_fill(mask[:, :k], -float("inf"))
    u = synthetic.uniforms24((B, k + 1), g, DEV)
    w = synthetic.Workload(synthetic.WORKLOADS[1], z, y, None, u, 1.0)
    for top_k, top_p in ((7, 1.0), (400, 1.0), (0, 0.83), (400, 0.61)):
        x = torch.from_numpy(truncated_drafts(f32(y), 1.0, top_k, top_p, 5)).to(DEV)
        check(sv, w, 1.0, x, top_k, top_p)


def test_top_k_one_is_greedy(sv):
    """top_k = 1 keeps only the row maximum on both sides: with the draft's
    argmax as its token, the rule commits exactly the greedy tokens."""
    B, k, V = 64, 6, 32000
    w = synthetic.chain(B, k, V, "fp32", seed=9, device=DEV)
    x = torch.argmax(w.draft.float(), dim=2).to(torch.int32)
    toks, na = sv.sample_truncated(w.target, w.draft, x, w.uniforms, w.T, 1, 1.0)
    gt, gn = sv.greedy(w.target, x)
    torch.cuda.synchronize()
    assert torch.equal(toks, gt) and torch.equal(na, gn)
    check(sv, w, w.T, x, 1, 1.0)


def test_truncation_off_is_plain_sampling(sv):
    w = synthetic.chain(32, 5, 32000, "bf16", seed=4, device=DEV)
    a = sv.sample_truncated(w.target, w.draft, w.tokens, w.uniforms, w.T, 0, 1.0, return_probs=True)
    b = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, return_probs=True)
    c = sv.sample_truncated(w.target, w.draft, w.tokens, w.uniforms, w.T, 32000, 1.5,
                            return_probs=True)
    torch.cuda.synchronize()
    for ta, tb, tc in zip(a, b, c):
        assert torch.equal(ta, tb) and torch.equal(tc, tb)


def test_truncated_deterministic(sv):
    w, T, x = workload(48, 6, 32000, "bf16", 31, 50, 0.9)
    r1 = sv.sample_truncated(w.target, w.draft, x, w.uniforms, T, 50, 0.9, return_probs=True)
    r2 = sv.sample_truncated(w.target, w.draft, x, w.uniforms, T, 50, 0.9, return_probs=True)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("cid,top_k,top_p", [(3, 0, 0.8), (5, 50, 0.9), (5, 0, 0.8), (2, 20, 1.0)])
def test_truncated_workload_subsets(sv, cid, top_k, top_p):
    """The workloads' own rows (vocabulary, dtype, temperature, spikes), a few
    sequences each."""
    cfg = synthetic.WORKLOADS[cid]
    B = 6
    w = synthetic.generate(cid, device=DEV, B=B)
    y = f32(w.draft)
    x = torch.from_numpy(truncated_drafts(y, w.T, top_k, top_p, cid)).to(DEV)
    rep, _, _ = check(sv, w, w.T, x, top_k, top_p)
    assert rep.rounds == B and cfg.V == w.target.shape[2]


def test_truncated_full_size_sampled(sv):
    """The 512 x 16 x 128256 bf16 workload at full size, top-p 0.8: every
    sequence's round is run and checked for the rule's invariants, and 64
    evenly spaced sequences (their drafts drawn from the truncated q') are
    checked against the oracle one by one."""
    w = synthetic.generate(5, device=DEV)
    B, k = w.tokens.shape
    idx = np.arange(0, B, 8)
    ti = torch.from_numpy(idx).to(DEV)
    x = w.tokens.clone()
    x[ti] = torch.from_numpy(truncated_drafts(f32(w.draft[ti]), w.T, 0, 0.8, 55)).to(DEV)
    toks, na = sv.sample_truncated(w.target, w.draft, x, w.uniforms, w.T, 0, 0.8)
    torch.cuda.synchronize()
    toks, na, xx = npi(toks), npi(na), npi(x)
    assert ((na >= 0) & (na <= k)).all()
    for b in range(B):
        assert (toks[b, :na[b]] == xx[b, :na[b]]).all()
        assert 0 <= toks[b, na[b]] < w.target.shape[2]
        assert (toks[b, na[b] + 1:] == -1).all()
    rep = parity.SampleReport()
    for c0 in range(0, idx.size, 16):
        sel = idx[c0:c0 + 16]
        ts = torch.from_numpy(sel).to(DEV)
        parity.check_sample_truncated(f32(w.target[ts]), f32(w.draft[ts]), xx[sel], npi(w.uniforms)[sel],
                                      w.T, 0, 0.8, toks[sel], na[sel], eps=EPS, report=rep, seq_ids=sel)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    assert rep.rounds == 64
    print(rep.summary())


def test_truncated_past_2_31_elements(sv):
    """Top-k 50 + top-p 0.8 on 1100 x 16 x 131072 target and 1100 x 15 x
    131072 draft logits (bf16), each tensor past 2^31 elements: target rows of
    sequences 1024.. and draft rows of sequences 1093.. start beyond element
    2^31; the sequences on either side are checked against the oracle."""
    B, k, V = 1100, 15, 131072
    w = synthetic.chain(B, k, V, "bf16", var_target=3.0, var_noise=1.0, seed=2 ** 31 + 1, device=DEV)
    assert w.target.numel() > 2 ** 31 and w.draft.numel() > 2 ** 31
    idx = np.array([0, 1, 1023, 1024, 1092, 1093, 1099])
    ti = torch.from_numpy(idx).to(DEV)
    x = w.tokens.clone()
    x[ti] = torch.from_numpy(truncated_drafts(f32(w.draft[ti]), w.T, 50, 0.8, 77)).to(DEV)
    toks, na = sv.sample_truncated(w.target, w.draft, x, w.uniforms, w.T, 50, 0.8)
    torch.cuda.synchronize()
    toks, na = npi(toks), npi(na)
    assert ((na >= 0) & (na <= k)).all()
    rep = parity.check_sample_truncated(f32(w.target[ti]), f32(w.draft[ti]), npi(x)[idx],
                                        npi(w.uniforms[ti]), w.T, 50, 0.8, toks[idx], na[idx],
                                        eps=EPS)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    print(rep.summary())
    del w, x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_truncated_many_equal_logits(sv, dtype):
    """16-bit rows with 65536 or more equal finite logits (the one-pass key
    histogram cannot hold that count and hands the row to the radix passes),
    +0.0 and -0.0 together past 65535, and rows with more than 65535 masked
    (-inf) tokens."""
    g = torch.Generator(device=DEV).manual_seed(8)
    B, k, V = 3, 2, 70001
    tdt = synthetic.DTYPES[dtype]
    z = torch.randn((B, k + 1, V), generator=g, device=DEV).to(tdt)
    y = torch.randn((B, k, V), generator=g, device=DEV).to(tdt)
    z[0, :, :66000] = 0.5                          # one value 66000 times
    y[0, :, 1000:67500] = -1.25
    zero = torch.rand((V,), generator=g, device=DEV) < 0.5
    z[1, :, :68000] = torch.where(zero[:68000], torch.tensor(0.0, dtype=tdt, device=DEV),
                                  torch.tensor(-0.0, dtype=tdt, device=DEV))
    z[2, :, 2:68002] = -float("inf")               # a masked row: 68000 -inf
    y[2, :, 5:68005] = -float("inf")
    u = synthetic.uniforms24((B, k + 1), g, DEV)
    w = synthetic.Workload(synthetic.WORKLOADS[1], z, y, None, u, 1.0)
    for top_k, top_p in ((100, 1.0), (0, 0.9), (70000, 0.5), (3, 0.99)):
        x = torch.from_numpy(truncated_drafts(f32(y), 1.0, top_k, top_p, 9)).to(DEV)
        check(sv, w, 1.0, x, top_k, top_p)


def small_top_k_rows(n, V, tdt, g):
    """n rows of V logits, one pattern per row (row i: pattern i % 12): plain
    normal; ascending and descending order (each new logit beats or trails
    every earlier one, the worst and best order for a streamed floor); all
    negative; 40 or 3 finite logits among -inf; 300 equal logits above the
    rest; one constant; a boundary among +0.0 and -0.0; logits near the
    format's largest magnitudes; every logit in a dozen values (ties
    everywhere); normal with one far spike."""
    big = 60000.0 if tdt == torch.float16 else 3.0e38
    rows = []
    for i in range(n):
        p = i % 12
        r = torch.randn((V,), generator=g, device=DEV)
        if p == 1:
            r = torch.sort(r).values
        elif p == 2:
            r = torch.sort(r, descending=True).values
        elif p == 3:
            r = r - 20.0
        elif p in (4, 5):
            keep = torch.randperm(V, generator=g, device=DEV)[:40 if p == 4 else 3]
            r = torch.full((V,), -float("inf"), device=DEV).index_put((keep,), r[keep])
        elif p == 6:
            r[torch.randperm(V, generator=g, device=DEV)[:300]] = 9.0
        elif p == 7:
            r = torch.full((V,), 1.5, device=DEV)
        elif p == 8:
            r = -torch.rand((V,), generator=g, device=DEV) - 0.5
            pos = torch.randperm(V, generator=g, device=DEV)
            r[pos[:20]] = torch.rand((20,), generator=g, device=DEV) + 1.0
            z = pos[20:20 + V // 3]
            r[z] = torch.where(torch.rand(z.shape, generator=g, device=DEV) < 0.5, 0.0, -0.0)
        elif p == 9:
            r = torch.sign(r) * big * (1.0 - 0.01 * torch.rand((V,), generator=g, device=DEV))
        elif p == 10:
            r = torch.randint(-6, 6, (V,), generator=g, device=DEV).float() * 0.5
        elif p == 11:
            r[int(torch.randint(V, (1,), generator=g, device=DEV))] = 25.0
        rows.append(r)
    return torch.stack(rows).to(tdt)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("V", [3001, 3004, 3005, 3007, 32000])
@pytest.mark.parametrize("B", [12, 40, 110])
def test_truncated_small_top_k_equals_fp32(sv, dtype, V, B):
    """Top-k up to 256: fp32 rows take the candidate lists (k_topk32), 16-bit
    rows the candidate lists (k_topk16) when they outnumber the compute units
    more than three times, else the histogram pass (k_trunc16).  On rows
    built to stress them (small_top_k_rows), at every top-k from 1 to 256
    (and 257) and top-p from off to 1e-6, the 16-bit result must equal, bit
    for bit, that of the same rows upcast to fp32; some settings are checked
    against the oracle too.  B = 12 gives 84 rows (1024 fp32 threads per
    row, or at V = 32000 its slices), B = 40 gives 280 rows (256 fp32
    threads per row), both k_trunc16 for 16-bit rows; B = 110 gives 770 rows,
    k_topk16's.  V = 3001, 3004, 3005 and 3007 end each row with a partial
    vector of 1, 4, 5 and 7 logits, taken after the stream by lanes whose
    lists may be nearly full (ascending rows)."""
    g = torch.Generator(device=DEV).manual_seed(V + B)
    tdt = synthetic.DTYPES[dtype]
    k = 3
    z = small_top_k_rows(B * (k + 1), V, tdt, g).view(B, k + 1, V)
    y = small_top_k_rows(B * k + 5, V, tdt, g)[5:].view(B, k, V)   # other patterns than z's rows
    u = synthetic.uniforms24((B, k + 1), g, DEV)
    tok = torch.randint(0, V, (B, k), generator=g, device=DEV, dtype=torch.int32)
    for top_k in (1, 2, 5, 39, 40, 41, 50, 63, 64, 65, 255, 256, 257):
        for top_p in (1.0, 0.9, 0.5, 1e-6):
            a = sv.sample_truncated(z, y, tok, u, 0.8, top_k, top_p, return_probs=True)
            b = sv.sample_truncated(z.float(), y.float(), tok, u, 0.8, top_k, top_p,
                                    return_probs=True)
            torch.cuda.synchronize()
            for ta, tb in zip(a, b):
                assert torch.equal(ta, tb), (top_k, top_p)
    w = synthetic.Workload(synthetic.WORKLOADS[1], z, y, None, u, 0.8)
    for top_k, top_p in ((3, 1.0), (40, 0.9), (256, 0.5)):
        x = torch.from_numpy(truncated_drafts(f32(y), 0.8, top_k, top_p, 13)).to(DEV)
        check(sv, w, 0.8, x, top_k, top_p)


@pytest.mark.parametrize("V", [3001, 3007, 32000])
@pytest.mark.parametrize("B", [12, 40])
def test_truncated_small_top_k_fp32(sv, V, B):
    """The fp32 candidate-list pass on fp32 values that no 16-bit format
    holds (small_top_k_rows in fp32: ties, -inf masks, +-0, magnitudes near
    3e38, ascending rows), against the oracle, with 1024 (B = 12) and 256
    (B = 40) threads per row; constant rows overflow the lists and take the
    radix passes."""
    g = torch.Generator(device=DEV).manual_seed(3 * V + B)
    k = 3
    z = small_top_k_rows(B * (k + 1), V, torch.float32, g).view(B, k + 1, V)
    y = small_top_k_rows(B * k + 5, V, torch.float32, g)[5:].view(B, k, V)
    u = synthetic.uniforms24((B, k + 1), g, DEV)
    w = synthetic.Workload(synthetic.WORKLOADS[1], z, y, None, u, 0.8)
    for top_k, top_p in ((1, 1.0), (5, 0.9), (50, 0.8), (63, 1.0), (64, 0.5), (256, 0.99)):
        x = torch.from_numpy(truncated_drafts(f32(y), 0.8, top_k, top_p, 17)).to(DEV)
        check(sv, w, 0.8, x, top_k, top_p)


@pytest.mark.parametrize("V", [3001, 32000, 40000])
def test_truncated_fp32_value_bins(sv, V):
    """fp32 rows under top-p alone, or a top-k beyond the candidate lists,
    are binned by value first and the boundary bin gathered (V <= 32768 from
    an LDS copy of the row, 40000 streamed): on rows built to stress it
    (small_top_k_rows), bf16 values upcast to fp32 must give, bit for bit,
    what the 16-bit histogram pass gives on the bf16 rows, at top-k 0, 257,
    300, 1000 and V - 1 with top-p from off to 1e-6; fp32-only rows are
    checked against the oracle.  Constant rows and a dozen repeated values
    leave boundary bins too full to gather (the radix passes take them);
    magnitudes near 3e38 make the bins' scale tiny."""
    g = torch.Generator(device=DEV).manual_seed(V + 77)
    B, k = 12, 3
    z = small_top_k_rows(B * (k + 1), V, torch.bfloat16, g).view(B, k + 1, V)
    y = small_top_k_rows(B * k + 5, V, torch.bfloat16, g)[5:].view(B, k, V)
    u = synthetic.uniforms24((B, k + 1), g, DEV)
    tok = torch.randint(0, V, (B, k), generator=g, device=DEV, dtype=torch.int32)
    for top_k in (0, 257, 300, 1000, V - 1):
        for top_p in (1.0, 0.9, 0.5, 1e-6):
            if top_k == 0 and top_p >= 1.0:
                continue
            a = sv.sample_truncated(z, y, tok, u, 0.8, top_k, top_p, return_probs=True)
            b = sv.sample_truncated(z.float(), y.float(), tok, u, 0.8, top_k, top_p, return_probs=True)
            torch.cuda.synchronize()
            for ta, tb in zip(a, b):
                assert torch.equal(ta, tb), (top_k, top_p)
    zf = small_top_k_rows(B * (k + 1), V, torch.float32, g).view(B, k + 1, V)
    yf = small_top_k_rows(B * k + 5, V, torch.float32, g)[5:].view(B, k, V)
    w = synthetic.Workload(synthetic.WORKLOADS[1], zf, yf, None, u, 0.8)
    for top_k, top_p in ((0, 0.8), (0, 1e-6), (300, 0.9), (1000, 1.0)):
        x = torch.from_numpy(truncated_drafts(f32(yf), 0.8, top_k, top_p, 19)).to(DEV)
        check(sv, w, 0.8, x, top_k, top_p)


@pytest.mark.parametrize("V", [32767, 32768, 32769])
@pytest.mark.parametrize("top_k,top_p", [(0, 0.9), (300, 0.9), (40, 0.9)])
def test_truncated_fp32_lds_boundary(sv, V, top_k, top_p):
    """Without a top-k of at most 256, fp32 rows of up to 32768 logits run the
    radix passes on an LDS copy and longer ones stream the row for every
    pass: both sides of the switch (top-k 40 takes the candidate lists)."""
    w, T, x = workload(3, 3, V, "fp32", V, top_k, top_p)
    check(sv, w, T, x, top_k, top_p)


def test_truncated_fp32_large_vocabulary(sv):
    """fp32 rows at V = 128256: top-k 50 takes the candidate lists, top-p
    alone the radix passes (three digits, the row streamed for each)."""
    w, T, x = workload(2, 2, 128256, "fp32", 61, 50, 0.8)
    check(sv, w, T, x, 50, 0.8)
    w, T, x = workload(2, 2, 128256, "fp32", 62, 0, 0.95)
    check(sv, w, T, x, 0, 0.95)


def sliced_rows(V, tdt, g):
    """Rows for the sliced pass (B = 1, k = 4): five target rows, then four
    draft rows.  Target: plain normal; 5000 logits tied at the top, spread
    over every slice (more candidates than the merge gathers); 100 distinct
    large logits over 600 tied just below them (at top-k 256 the kept tie
    group outgrows the merge); the first half masked (whole slices with no
    finite logit); ten finite logits, all in the last 300 (the last slice and
    its partial vector).  Draft: normal; ascending (the largest in the last
    slice); a dozen values (ties everywhere); one finite logit."""
    n = torch.randn((9, V), generator=g, device=DEV)
    z = n[:5].clone()
    z[1, torch.arange(0, V, V // 5000, device=DEV)[:5000]] = 8.0
    z[2] = z[2] - 5.0
    p = torch.randperm(V, generator=g, device=DEV)
    z[2, p[:100]] = 10.0 + 4.0 * torch.rand((100,), generator=g, device=DEV)
    z[2, p[100:700]] = 9.0
    z[3, :V // 2] = -float("inf")
    last = V - 300 + torch.randperm(300, generator=g, device=DEV)[:10]
    keep = z[4, last].clone()
    z[4] = -float("inf")
    z[4, last] = keep
    y = n[5:].clone()
    y[1] = torch.sort(y[1]).values
    y[2] = torch.randint(-6, 6, (V,), generator=g, device=DEV).float() * 0.5
    one = int(torch.randint(V, (1,), generator=g, device=DEV))
    y[3] = -float("inf")
    y[3, one] = 1.0
    return z.to(tdt).view(1, 5, V), y.to(tdt).view(1, 4, V)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_truncated_sliced_rows(sv, dtype):
    """B = 1 at V = 128259: fp32 rows are cut into 31 slices, summarised apart
    and merged per row; 16-bit rows take the histogram pass.  Against the
    oracle on rows built to reach the merge's limits (sliced_rows), and bit
    for bit against the same sequence verified inside a batch of 100, whose
    900 rows take the candidate lists whole (one workgroup per row)."""
    V = 128259
    g = torch.Generator(device=DEV).manual_seed(59)
    tdt = synthetic.DTYPES[dtype]
    z, y = sliced_rows(V, tdt, g)
    u = synthetic.uniforms24((1, 5), g, DEV)
    w = synthetic.Workload(synthetic.WORKLOADS[1], z, y, None, u, 0.9)
    # the batch of 100: this sequence first, plain normal rows after it
    NB = 100
    zb = torch.randn((NB, 5, V), generator=g, device=DEV).to(tdt)
    yb = torch.randn((NB, 4, V), generator=g, device=DEV).to(tdt)
    zb[0], yb[0] = z[0], y[0]
    ub = synthetic.uniforms24((NB, 5), g, DEV)
    ub[0] = u[0]
    for top_k, top_p in ((50, 1.0), (256, 0.9), (5, 0.5)):
        x = torch.from_numpy(truncated_drafts(f32(y), 0.9, top_k, top_p, 23)).to(DEV)
        check(sv, w, 0.9, x, top_k, top_p)
        xb = torch.randint(0, V, (NB, 4), generator=g, device=DEV, dtype=torch.int32)
        xb[0] = x[0]
        a = sv.sample_truncated(z, y, x, u, 0.9, top_k, top_p, return_probs=True)
        b = sv.sample_truncated(zb, yb, xb, ub, 0.9, top_k, top_p, return_probs=True)
        torch.cuda.synchronize()
        for ta, tb in zip(a, b):
            assert torch.equal(ta[0], tb[0]), (top_k, top_p)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_truncated_k63(sv, dtype):
    """The longest draft one wave decides (k = 63)."""
    w, T, x = workload(3, 63, 1000, dtype, 63, 10, 0.9)
    check(sv, w, T, x, 10, 0.9)


# ---------------------------------------------------------------------------
# a seeded sweep over random shapes, dtypes, scales and truncation settings
# ---------------------------------------------------------------------------
def random_trunc_case(i):
    """Case i: log-uniform V in [1, 70000], k up to 31, temperatures 0.1-3,
    logit variances 0.5-100, top-k from off to V-1 and top-p from off to
    1e-6; the oracle's work is capped at 2e6 elements per case."""
    r = np.random.default_rng(5000 + i)
    dtype = ["fp32", "fp16", "bf16"][int(r.integers(3))]
    k = int(r.choice([1, 2, 4, 8, 16, 31]))
    V = max(1, int(np.exp(r.uniform(0.0, np.log(70000.0)))))
    B = int(r.integers(1, 17))
    while B > 1 and B * (2 * k + 1) * V > 2_000_000:
        B //= 2
    V = min(V, max(1, 2_000_000 // (B * (2 * k + 1))))
    T = float(np.exp(r.uniform(np.log(0.1), np.log(3.0))))
    var_t = float(r.choice([0.5, 2.0, 9.0, 100.0]))
    top_k = int(r.choice([0, 1, 2, 5, 50, 1000, max(1, V - 1)]))
    top_p = float(r.choice([1.0, 0.999, 0.9, 0.5, 0.1, 1e-6]))
    return dtype, B, k, V, T, var_t, top_k, top_p


@pytest.mark.parametrize("i", range(16))
def test_random_truncated_cases(sv, i):
    dtype, B, k, V, T, var_t, top_k, top_p = random_trunc_case(i)
    print(f"case {i}: {dtype} B={B} k={k} V={V} T={T:.3f} var={var_t} top_k={top_k} top_p={top_p}",
          flush=True)
    w = synthetic.chain(B, k, V, dtype, var_target=var_t, var_noise=0.3 * var_t, T=T, seed=6000 + i,
                        device=DEV)
    x = torch.from_numpy(truncated_drafts(f32(w.draft), T, top_k, top_p, 6000 + i)).to(DEV)
    check(sv, w, T, x, top_k, top_p)


def random_small_top_k_case(i):
    """Case i of the candidate-list sweep: fp16 or bf16, V in [8, 200000]
    (log-uniform, so every partial-vector length occurs), top-k uniform in
    [1, 256], top-p from off to 1e-6, and one of four value laws: Gaussian
    logits of variance 0.5-100, a dozen distinct values (ties everywhere),
    Gaussian logits with a quarter masked to -inf, or a shuffled ramp (every
    logit distinct, a flat distribution)."""
    r = np.random.default_rng(7000 + i)
    dtype = ["fp16", "bf16"][int(r.integers(2))]
    V = int(np.exp(r.uniform(np.log(8.0), np.log(200000.0))))
    # even cases: few rows (k_trunc16 for 16-bit, slices for long fp32 rows);
    # odd: 780 rows (k_topk16, 256 fp32 threads per row)
    rows = int(max(1, min(24, 3_000_000 // V))) if i % 2 == 0 else 780
    top_k = int(r.integers(1, 257))
    top_p = float(r.choice([1.0, 0.999, 0.9, 0.5, 0.1, 1e-6]))
    law = int(r.integers(4))
    scale = float(np.sqrt(r.choice([0.5, 2.0, 9.0, 100.0])))
    return dtype, V, rows, top_k, top_p, law, scale


@pytest.mark.parametrize("i", range(24))
def test_random_small_top_k_equals_fp32(sv, i):
    """The candidate-list pass for 16-bit rows against the one for fp32 rows
    on the same (upcast) rows, bit for bit, over a seeded sweep of shapes,
    settings and value laws (random_small_top_k_case)."""
    dtype, V, rows, top_k, top_p, law, scale = random_small_top_k_case(i)
    print(f"case {i}: {dtype} V={V} rows={rows} top_k={top_k} top_p={top_p} law={law} scale={scale:.2f}",
          flush=True)
    g = torch.Generator(device=DEV).manual_seed(7000 + i)
    tdt = synthetic.DTYPES[dtype]
    B, k = max(1, rows // 3), 1                    # rows = B * (2k + 1)
    n = B * (2 * k + 1)
    if law == 0:
        z = torch.randn((n, V), generator=g, device=DEV) * scale
    elif law == 1:
        z = torch.randint(-6, 6, (n, V), generator=g, device=DEV).float() * 0.5
    elif law == 2:
        z = torch.randn((n, V), generator=g, device=DEV) * scale
        z = z.masked_fill(torch.rand((n, V), generator=g, device=DEV) < 0.25, -float("inf"))
        z[:, 0] = 0.0                                 # at least one finite logit per row
    else:
        ramp = torch.linspace(-4.0, 4.0, V, device=DEV)
        z = torch.stack([ramp[torch.randperm(V, generator=g, device=DEV)] for _ in range(n)])
    z = z.to(tdt)
    tgt = z[:B * (k + 1)].view(B, k + 1, V)
    dft = z[B * (k + 1):].view(B, k, V)
    u = synthetic.uniforms24((B, k + 1), g, DEV)
    tok = torch.randint(0, V, (B, k), generator=g, device=DEV, dtype=torch.int32)
    a = sv.sample_truncated(tgt, dft, tok, u, 1.0, top_k, top_p, return_probs=True)
    b = sv.sample_truncated(tgt.float(), dft.float(), tok, u, 1.0, top_k, top_p, return_probs=True)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)
