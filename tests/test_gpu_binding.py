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
