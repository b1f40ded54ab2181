"""The entry points under HIP graph capture: nothing they enqueue allocates,
sets memory with a memset, or synchronises, so a caller can capture a call
into a graph and replay it on new inputs.  Each replay here runs on inputs
copied into the captured buffers, with eager work and synchronisations in
between, and must equal an eager call on the same inputs bit for bit.  Calls
on several streams with their own workspaces may also overlap."""
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


def chain_sets(n, B, k, V, dtype):
    return [synthetic.chain(B, k, V, dtype, var_target=3.0, var_noise=2.0, spike=6.0,
                            seed=100 + s, device=DEV) for s in range(n)]


def capture(run):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                          # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    return g, outs


def replay_and_compare(g, outs, load, eager, n):
    for i in range(1, n):
        load(i)
        junk = torch.randn(1 << 20, device=DEV)          # eager work between replays
        _ = float(junk.abs().max())
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        ref = eager(i)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), (i, a, b)


@pytest.mark.parametrize("mode", ["sample", "greedy", "sample_lazy", "greedy_lazy", "truncated",
                                  "truncated_top_p", "lenient"])
@pytest.mark.parametrize("B,k,V,dtype", [(64, 6, 32000, "bf16"), (4, 4, 32000, "fp32"), (8, 4, 32000, "fp16")])
def test_chain_entry_points_replay(sv, mode, B, k, V, dtype):
    """B = 64: the draw in a kernel of its own, and 832 16-bit rows, which
    top-k 20 sends to the candidate lists (top-p alone: the histogram pass).
    B = 4 (64 chunk workgroups) and B = 8 (128, the most for which the chunk
    pass makes the draw itself): the per-sequence counters must start every
    replay at zero, cleared by the first kernel (no memset is captured).
    B = 4's 36 fp32 rows take the candidate lists cut into slices and merged
    (top-k 20) and the value bins from LDS (top-p alone); B = 8's 72 fp16
    rows the histogram pass."""
    sets = chain_sets(4, B, k, V, dtype)
    tgt = sets[0].target.clone()
    dft = sets[0].draft.clone()
    x = sets[0].tokens.clone()
    u = sets[0].uniforms.clone()
    T = sets[0].T
    ws = torch.empty(sv.workspace_bytes(B, 2 * k + 1, V, tgt.dtype), dtype=torch.uint8, device=DEV)
    out_t = torch.empty((B, k + 1), dtype=torch.int32, device=DEV)
    out_n = torch.empty(B, dtype=torch.int32, device=DEV)

    def call(t, d, xx, uu, workspace, ot=None, on=None):
        if mode == "sample":
            return sv.sample(t, d, xx, uu, T, out_tokens=ot, out_num_accepted=on, workspace=workspace)
        if mode == "greedy":
            return sv.greedy(t, xx, out_tokens=ot, out_num_accepted=on, workspace=workspace)
        if mode == "sample_lazy":
            return sv.sample_lazy(t, d, xx, uu, T, out_tokens=ot, out_num_accepted=on,
                                  workspace=workspace)
        if mode == "greedy_lazy":
            return sv.greedy_lazy(t, xx, out_tokens=ot, out_num_accepted=on, workspace=workspace)
        if mode == "truncated":        # the candidate-list pass
            return sv.sample_truncated(t, d, xx, uu, T, 20, 0.9, workspace=workspace)
        if mode == "truncated_top_p":  # the pattern-histogram pass
            return sv.sample_truncated(t, d, xx, uu, T, 0, 0.9, workspace=workspace)
        return sv.sample_lenient(t, d, xx, uu, T, 2.0, workspace=workspace)

    def run():
        r = call(tgt, dft, x, u, ws, out_t, out_n)
        return r if mode in ("truncated", "truncated_top_p", "lenient") else (out_t, out_n)

    def load(i):
        tgt.copy_(sets[i].target)
        dft.copy_(sets[i].draft)
        x.copy_(sets[i].tokens)
        u.copy_(sets[i].uniforms)

    def eager(i):
        w = sets[i]
        return call(w.target, w.draft, w.tokens, w.uniforms, None)

    g, outs = capture(run)
    replay_and_compare(g, outs, load, eager, len(sets))


def test_candidates_replay(sv):
    sets = [synthetic.candidates(8, 8, 8, 8, 4096, seed=200 + s, device=DEV) for s in range(4)]
    B, C, R, V = sets[0].target.shape
    L = sets[0].tokens.shape[2]
    tgt = sets[0].target.clone()
    cand = sets[0].tokens.clone()
    ws = torch.empty(sv.workspace_bytes(B, C * R, V, tgt.dtype), dtype=torch.uint8, device=DEV)
    out = (torch.empty((B, L + 1), dtype=torch.int32, device=DEV),
           torch.empty(B, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV))

    def run():
        sv.greedy_candidates(tgt, cand, out_tokens=out[0], out_num_accepted=out[1], out_best=out[2],
                             workspace=ws)
        return out

    def load(i):
        tgt.copy_(sets[i].target)
        cand.copy_(sets[i].tokens)

    def eager(i):
        return sv.greedy_candidates(sets[i].target, sets[i].tokens)

    g, outs = capture(run)
    replay_and_compare(g, outs, load, eager, len(sets))


def test_calls_on_concurrent_streams(sv):
    """Calls on different streams with their own workspaces may overlap: four
    streams, each with its own inputs, launched back to back with no
    synchronisation in between, equal the same calls made one at a time."""
    B, k, V = 96, 8, 32000
    sets = chain_sets(4, B, k, V, "bf16")
    streams = [torch.cuda.Stream() for _ in sets]
    wss = [torch.empty(sv.workspace_bytes(B, 2 * k + 1, V, torch.bfloat16), dtype=torch.uint8, device=DEV)
           for _ in sets]
    ref = []
    for w in sets:
        ref.append(sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, return_probs=True))
        ref.append(sv.greedy(w.target, w.tokens))
    torch.cuda.synchronize()
    got = [None] * len(ref)
    for rep in range(3):
        for i, (w, s, ws) in enumerate(zip(sets, streams, wss)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                got[2 * i] = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, return_probs=True,
                                       workspace=ws, stream=s)
        for i, (w, s, ws) in enumerate(zip(sets, streams, wss)):
            with torch.cuda.stream(s):
                got[2 * i + 1] = sv.greedy(w.target, w.tokens, workspace=ws, stream=s)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            for x, y in zip(a, b):
                assert torch.equal(x, y), rep
