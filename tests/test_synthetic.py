"""The seeded input generator, on the CPU: shapes and dtypes of every
workload, determinism, the uniforms' grid, the candidate layout and its
token-tree form.  The generator holds none of the rule's arithmetic; these
tests only fix what the parity tests and bench.py rely on it for."""
import numpy as np
import pytest
import torch

import synthetic

DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_chain_workload_shapes(cid):
    cfg = synthetic.WORKLOADS[cid]
    B, V = min(cfg.B, 3), 1000
    w = synthetic.generate(cid, B=B, V=V)
    k = cfg.k
    assert w.target.shape == (B, k + 1, V) and w.target.dtype == DT[cfg.dtype]
    assert w.draft.shape == (B, k, V) and w.draft.dtype == DT[cfg.dtype]
    assert w.tokens.shape == (B, k) and w.tokens.dtype == torch.int32
    assert w.uniforms.shape == (B, k + 1) and w.uniforms.dtype == torch.float32
    assert ((w.tokens >= 0) & (w.tokens < V)).all()
    assert torch.isfinite(w.target.float()).all() and torch.isfinite(w.draft.float()).all()
    assert w.T == cfg.T


def test_candidate_workload_shapes_and_shared_rows():
    cfg = synthetic.WORKLOADS[4]
    w = synthetic.generate(4, B=2, V=500)
    assert w.target.shape == (2, cfg.C, cfg.R, 500) and w.target.dtype == torch.bfloat16
    assert w.tokens.shape == (2, cfg.C, cfg.L) and w.draft is None
    # the first shared_rows rows are the same for every candidate of a sequence
    S = cfg.shared_rows
    for c in range(1, cfg.C):
        assert torch.equal(w.target[:, c, :S], w.target[:, 0, :S])
    assert not torch.equal(w.target[:, 1, S], w.target[:, 0, S])


def test_token_tree_maps_every_candidate_row():
    w = synthetic.candidates(3, 4, 5, 6, 200, shared_rows=2, seed=5)
    nodes, rows = synthetic.as_tree(w)
    B, C, R, V = w.target.shape
    assert nodes.shape == (B, 2 + C * (R - 2), V) and rows.shape == (B, C, R)
    for b in range(B):
        for c in range(C):
            for i in range(R):
                assert torch.equal(nodes[b, rows[b, c, i]], w.target[b, c, i])


def test_generation_is_deterministic_per_seed_and_set():
    a = synthetic.generate(2, B=2, V=300)
    b = synthetic.generate(2, B=2, V=300)
    c = synthetic.generate(2, B=2, V=300, set_index=1)
    for x, y in [(a.target, b.target), (a.draft, b.draft), (a.tokens, b.tokens), (a.uniforms, b.uniforms)]:
        assert torch.equal(x, y)
    assert not torch.equal(a.target, c.target) and not torch.equal(a.uniforms, c.uniforms)


def test_uniforms_lie_on_the_2_24_grid_below_one():
    g = synthetic.make_generator(7, "cpu")
    u = synthetic.uniforms24((100000,), g, "cpu").numpy().astype(np.float64)
    assert u.min() >= 0.0 and u.max() < 1.0
    m = u * 2 ** 24
    assert np.array_equal(m, np.round(m))
    assert abs(u.mean() - 0.5) < 0.01


def test_draft_is_the_target_plus_noise():
    """y = z + N(0, var_noise) before rounding: the draft rows follow the
    target rows (the correlation that sets the acceptance rate)."""
    w = synthetic.chain(4, 3, 5000, "fp32", var_target=2.0, var_noise=0.5, seed=3)
    d = (w.draft - w.target[:, :3]).numpy()
    assert abs(d.var() - 0.5) < 0.05 and abs(d.mean()) < 0.05
    assert abs(w.target.numpy().var() - 2.0) < 0.1
