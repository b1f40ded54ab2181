"""spec_verify_sample_noalloc, the entry point for callers that cannot
allocate, through the C ABI on the GPU: its results equal spec_verify_sample's
bit for bit and pass the oracle's bar, on two calls in a row (the second with
a smaller input, which finds the first call's contents in the shared static
scratch) issued back to back on one stream."""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from oracle import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = 1e-5
DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    import draft_verification_verify_amd as m
    return m


def outputs(w, fill=-5):
    B, k = w.tokens.shape
    return (torch.full((B, k + 1), fill, dtype=torch.int32, device=DEV),
            torch.full((B,), fill, dtype=torch.int32, device=DEV),
            torch.full((B, k), -1.0, dtype=torch.float32, device=DEV),
            torch.full((B, k), -1.0, dtype=torch.float32, device=DEV))


def call_noalloc(sv, w, outs, stream=None):
    """The raw C entry point, with the tensors' device pointers."""
    B, k = w.tokens.shape
    V = w.target.shape[2]
    st = (stream or torch.cuda.current_stream()).cuda_stream
    return sv.lib().spec_verify_sample_noalloc(
        w.target.data_ptr(), w.target.stride(1), w.draft.data_ptr(), w.draft.stride(1),
        w.tokens.data_ptr(), w.uniforms.data_ptr(), float(w.T), B, k, V, DT[w.target.dtype],
        outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(), st)


def check_against_sample_and_oracle(sv, w, outs, every=1):
    ref = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T, return_probs=True)
    torch.cuda.synchronize()
    for a, b in zip(ref, outs):
        assert torch.equal(a, b)
    B = w.tokens.shape[0]
    idx = np.arange(0, B, every)
    ti = torch.from_numpy(idx).to(DEV)
    z, y = w.target[ti].float().cpu().numpy(), w.draft[ti].float().cpu().numpy()
    x, u = w.tokens[ti].cpu().numpy(), w.uniforms[ti].cpu().numpy()
    rep = parity.check_sample(z, y, x, u, w.T, outs[0][ti].cpu().numpy(), outs[1][ti].cpu().numpy(),
                              eps=EPS, seq_ids=idx)
    assert rep.ok(), (rep.summary(), rep.failures[:3])
    worst = parity.check_probs(z, y, x, w.T, outs[2][ti].cpu().numpy(), outs[3][ti].cpu().numpy())
    assert worst <= EPS, worst
    return rep


def test_two_calls_in_a_row_second_smaller(sv):
    """B = 512, k = 16, V = 128256 bf16 (0.86 MiB of scratch), then at once
    B = 7, k = 5, V = 32003 fp16 (a ragged row, unaligned rows) on the same
    stream with no synchronisation between them."""
    big = synthetic.generate(5, device=DEV)
    small = synthetic.chain(7, 5, 32003, "fp16", var_target=3.0, var_noise=1.0, seed=77, device=DEV)
    ob, os_ = outputs(big), outputs(small)
    torch.cuda.synchronize()
    assert call_noalloc(sv, big, ob) == sv.SV_OK
    assert call_noalloc(sv, small, os_) == sv.SV_OK
    torch.cuda.synchronize()
    print("noalloc, workload 5:", check_against_sample_and_oracle(sv, big, ob, every=8).summary())
    print("noalloc, small:", check_against_sample_and_oracle(sv, small, os_).summary())


def test_side_stream_and_refusals(sv):
    """On a side stream of the current device it gives the same results; a
    shape beyond the scratch is refused with SV_ESCRATCH and leaves the
    outputs untouched; so is a bad argument (SV_EINVAL)."""
    w = synthetic.chain(16, 4, 20000, "bf16", seed=31, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = outputs(w)
    assert call_noalloc(sv, w, outs, stream=s) == sv.SV_OK
    s.synchronize()
    check_against_sample_and_oracle(sv, w, outs)

    outs = outputs(w, fill=-9)
    L = sv.lib()
    B, k = w.tokens.shape
    st = torch.cuda.current_stream().cuda_stream
    big_B = 4096                                   # 4096 x 33 rows of 128256: past 4 MiB of scratch
    assert L.spec_verify_workspace_bytes(big_B, 2 * 16 + 1, 128256, 2) > sv.NOALLOC_SCRATCH_BYTES
    assert L.spec_verify_sample_noalloc(w.target.data_ptr(), 128256, w.draft.data_ptr(), 128256,
                                        w.tokens.data_ptr(), w.uniforms.data_ptr(), 1.0, big_B, 16, 128256,
                                        2, outs[0].data_ptr(), outs[1].data_ptr(), None, None,
                                        st) == sv.SV_ESCRATCH
    assert L.spec_verify_sample_noalloc(w.target.data_ptr(), w.target.stride(1), w.draft.data_ptr(),
                                        w.draft.stride(1), w.tokens.data_ptr(), w.uniforms.data_ptr(),
                                        -1.0, B, k, 20000, 2, outs[0].data_ptr(), outs[1].data_ptr(),
                                        None, None, st) == sv.SV_EINVAL
    torch.cuda.synchronize()
    assert (outs[0] == -9).all() and (outs[1] == -9).all()


def test_binding(sv):
    """The binding's sample_noalloc equals sample."""
    w = synthetic.chain(9, 8, 12345, "fp32", seed=5, device=DEV)
    B, k = w.tokens.shape
    t = torch.empty((B, k + 1), dtype=torch.int32, device=DEV)
    n = torch.empty((B,), dtype=torch.int32, device=DEV)
    sv.sample_noalloc(w.target, w.draft, w.tokens, w.uniforms, w.T, out_tokens=t, out_num_accepted=n)
    a, b = sv.sample(w.target, w.draft, w.tokens, w.uniforms, w.T)
    torch.cuda.synchronize()
    assert torch.equal(a, t) and torch.equal(b, n)
