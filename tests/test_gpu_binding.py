"""The Python binding refuses tensors that do not match what an entry point
reads or writes (device, dtype, shape, layout) before any launch: the C ABI
takes plain pointers and cannot check buffer sizes itself."""
import os

import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    import draft_verification_verify_amd as m
    return m


@pytest.fixture(scope="module")
def w():
    return synthetic.chain(4, 3, 1000, "bf16", seed=3, device=DEV)


def bad_variants(t):
    """Wrong dtype, wrong shape, non-contiguous, on the CPU."""
    out = [t.to(torch.int64) if t.dtype == torch.int32 else t.to(torch.float64),
           t[..., :-1].contiguous(),
           torch.cat([t, t], dim=-1)[..., ::2],
           t.cpu()]
    return out


def test_sample_rejects_mismatched_inputs(sv, w):
    base = dict(target=w.target, draft=w.draft, draft_tokens=w.tokens, uniforms=w.uniforms)
    out_t = torch.full((4, 4), 7, dtype=torch.int32, device=DEV)
    for name in ("draft_tokens", "uniforms"):
        for bad in bad_variants(base[name]):
            args = dict(base, **{name: bad})
            with pytest.raises((ValueError, TypeError)):
                sv.sample(args["target"], args["draft"], args["draft_tokens"], args["uniforms"], 1.0,
                          out_tokens=out_t)
    for bad in (w.draft[:, :2], w.draft.float(), w.draft.cpu()):
        with pytest.raises((ValueError, TypeError)):
            sv.sample(w.target, bad, w.tokens, w.uniforms, 1.0, out_tokens=out_t)
    with pytest.raises(ValueError):
        sv.sample(w.target, w.draft, w.tokens, w.uniforms, 1.0,
                  out_tokens=torch.empty((4, 3), dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        sv.sample(w.target, w.draft, w.tokens, w.uniforms, 1.0, workspace=torch.empty(16, device="cpu"))
    torch.cuda.synchronize()
    assert (out_t == 7).all()          # nothing ran


def test_other_entry_points_reject_mismatched_tokens(sv, w):
    x64 = w.tokens.to(torch.int64)
    short = w.tokens[:, :2].contiguous()
    for bad in (x64, short, w.tokens.cpu()):
        for fn in (lambda x: sv.greedy(w.target, x), lambda x: sv.greedy_ext(w.target, x),
                   lambda x: sv.greedy_lazy(w.target, x),
                   lambda x: sv.sample_lazy(w.target, w.draft, x, w.uniforms, 1.0),
                   lambda x: sv.sample_lenient(w.target, w.draft, x, w.uniforms, 1.0, 2.0),
                   lambda x: sv.sample_truncated(w.target, w.draft, x, w.uniforms, 1.0, 5, 0.9)):
            with pytest.raises(ValueError):
                fn(bad)
    c = synthetic.candidates(2, 4, 4, 4, 500, "bf16", seed=5, device=DEV)
    for bad in (c.tokens.to(torch.int64), c.tokens[:, :, :2], c.tokens[:1].contiguous()):
        with pytest.raises(ValueError):
            sv.greedy_candidates(c.target, bad)
        with pytest.raises(ValueError):
            sv.greedy_candidates_ext(c.target, bad)
    with pytest.raises(TypeError):
        sv.greedy(w.target.to(torch.float64), w.tokens)


def test_a_float_workspace_counts_its_bytes(sv, w):
    """A workspace of another dtype is measured in bytes, not elements."""
    need = sv.workspace_bytes(4, 2 * 3 + 1, 1000, torch.bfloat16)
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=DEV)
    a = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, workspace=ws)
    b = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_batch_returns_empty_outputs(sv):
    """B = 0: nothing to verify, so every entry point returns empty outputs
    of the right shapes (the C ABI itself rejects B = 0)."""
    k, V = 3, 1000
    z = torch.zeros((0, k + 1, V), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((0, k, V), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((0, k), dtype=torch.int32, device=DEV)
    u = torch.zeros((0, k + 1), dtype=torch.float32, device=DEV)
    shapes = lambda outs: [tuple(o.shape) for o in outs]
    assert shapes(sv.greedy(z, x)) == [(0, k + 1), (0,)]
    assert shapes(sv.greedy_lazy(z, x)) == [(0, k + 1), (0,)]
    assert shapes(sv.greedy_ext(z, x)) == [(0, k + 1), (0,), (0, k + 1), (0,), (0,)]
    assert shapes(sv.sample(z, y, x, u, 1.0)) == [(0, k + 1), (0,)]
    assert shapes(sv.sample(z, y, x, u, 1.0, return_probs=True)) == [(0, k + 1), (0,), (0, k), (0, k)]
    assert shapes(sv.sample_lazy(z, y, x, u, 1.0)) == [(0, k + 1), (0,)]
    assert shapes(sv.sample_lenient(z, y, x, u, 1.0, 2.0)) == [(0, k + 1), (0,)]
    assert shapes(sv.sample_truncated(z, y, x, u, 1.0, 5, 0.9, return_probs=True)) == \
        [(0, k + 1), (0,), (0, k), (0, k)]
    C, L, R = 2, 4, 5
    t = torch.zeros((0, C, R, V), dtype=torch.bfloat16, device=DEV)
    ct = torch.zeros((0, C, L), dtype=torch.int32, device=DEV)
    assert shapes(sv.greedy_candidates(t, ct)) == [(0, L + 1), (0,), (0,)]
    assert shapes(sv.greedy_candidates_ext(t, ct)) == [(0, L + 1), (0,), (0,), (0, C, R)]
    n = torch.zeros((0, 7, V), dtype=torch.bfloat16, device=DEV)
    cr = torch.zeros((0, C, R), dtype=torch.int32, device=DEV)
    assert shapes(sv.greedy_tree(n, ct, cr)) == [(0, L + 1), (0,), (0,)]


def test_explicit_stream(sv, w):
    """A caller's stream on the logits' device is used as given."""
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())     # the inputs were written on the default stream
    a = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, stream=s)
    s.synchronize()
    b = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("entry", ["sample", "greedy"])
def test_stream_keeps_binding_buffers_alive(sv, w, entry):
    """With stream=s other than the current stream, the buffers the binding
    allocates (workspace, outputs) come from the current stream's pool while
    the kernels run on s.  They are recorded on s, so while s's work is still
    pending the caching allocator hands none of their memory to new
    allocations on the current stream, which are written at once with no
    synchronisation; the results equal a plain call's."""
    L = sv.lib()
    name = "spec_verify_" + entry
    orig = getattr(L, name)
    seen = {}

    def spy(*args):
        seen["ws"], seen["wsb"] = args[-3], args[-2]
        return orig(*args)

    def call(**kw):
        if entry == "sample":
            return sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, **kw)
        return sv.greedy(w.target, w.tokens, **kw)

    ref = [t.clone() for t in call()]
    torch.cuda.synchronize()
    a = torch.randn(8192, 8192, device=DEV)
    b = torch.empty_like(a)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                     # keeps s busy for tens of milliseconds
        for _ in range(6):
            torch.mm(a, a, out=b)
    setattr(L, name, spy)
    try:
        got = call(stream=s)
    finally:
        setattr(L, name, orig)
    live = {t.data_ptr() for t in got} | {seen["ws"]}
    junk = [torch.full((seen["wsb"],), 255, dtype=torch.uint8, device=DEV) for _ in range(4)]
    junk += [torch.full(t.shape, -7, dtype=t.dtype, device=DEV) for t in got]
    assert not live & {j.data_ptr() for j in junk}
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
