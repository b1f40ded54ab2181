"""Python binding of libspecverify.so, the MI355X speculative-decoding
verification library.

Argument marshalling only: every step of the verification runs in the HIP
kernels behind the C ABI declared in ``include/spec_verify.h``.  PyTorch
provides device memory (tensors) and streams.  There is no fallback: if the
library is not built, importing this package raises.  An empty batch (B = 0)
has nothing to verify: its (empty) outputs are returned without a call.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads torch's HIP runtime first, so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_EINVAL, SV_EDTYPE, SV_EWORKSPACE, SV_EHIP, SV_ESCRATCH = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 4 << 20        # SV_NOALLOC_SCRATCH_BYTES
SV_F32, SV_F16, SV_BF16 = 0, 1, 2
MAX_K = 63

_DTYPE = {torch.float32: SV_F32, torch.float16: SV_F16, torch.bfloat16: SV_BF16}


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {lib().spec_verify_status_string(status).decode()}")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libspecverify.so is not built ({LIB_PATH}); run __graft_entry__.build()")

_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(LIB_PATH)
        P, I, LL, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_size_t
        L.spec_verify_version.restype = I
        L.spec_verify_status_string.argtypes = [I]
        L.spec_verify_status_string.restype = ctypes.c_char_p
        L.spec_verify_workspace_bytes.argtypes = [I, I, I, I]
        L.spec_verify_workspace_bytes.restype = SZ
        L.spec_verify_greedy.argtypes = [P, LL, P, I, I, I, I, P, P, P, SZ, P]
        L.spec_verify_greedy.restype = I
        L.spec_verify_sample.argtypes = [P, LL, P, LL, P, P, F, I, I, I, I, P, P, P, P, P, SZ, P]
        L.spec_verify_sample.restype = I
        L.spec_verify_greedy_candidates.argtypes = [P, LL, P, I, I, I, I, I, I, P, P, P, P, SZ, P]
        L.spec_verify_greedy_candidates.restype = I
        L.spec_verify_greedy_ext.argtypes = [P, LL, P, I, I, I, I, P, P, P, P, P, P, SZ, P]
        L.spec_verify_greedy_ext.restype = I
        L.spec_verify_sample_lenient.argtypes = [P, LL, P, LL, P, P, F, F, I, I, I, I, P, P, P, P, P, SZ, P]
        L.spec_verify_sample_lenient.restype = I
        L.spec_verify_greedy_candidates_ext.argtypes = [P, LL, P, I, I, I, I, I, I, P, P, P, P, P, SZ, P]
        L.spec_verify_greedy_candidates_ext.restype = I
        L.spec_verify_greedy_tree.argtypes = [P, LL, I, P, P, I, I, I, I, I, I, P, P, P, P, SZ, P]
        L.spec_verify_greedy_tree.restype = I
        L.spec_verify_sample_lazy.argtypes = [P, LL, P, LL, P, P, F, I, I, I, I, P, P, P, SZ, P]
        L.spec_verify_sample_lazy.restype = I
        L.spec_verify_greedy_lazy.argtypes = [P, LL, P, I, I, I, I, P, P, P, SZ, P]
        L.spec_verify_greedy_lazy.restype = I
        L.spec_verify_sample_truncated.argtypes = [P, LL, P, LL, P, P, F, I, F, I, I, I, I, P, P, P,
                                                   P, P, SZ, P]
        L.spec_verify_sample_truncated.restype = I
        L.spec_verify_sample_noalloc.argtypes = [P, LL, P, LL, P, P, F, I, I, I, I, P, P, P, P, P]
        L.spec_verify_sample_noalloc.restype = I
        L.spec_verify_sample_timed.argtypes = [P, LL, P, LL, P, P, F, F, I, F, I, I, I, I, P, P, P, P,
                                               P, SZ, P, P, P]
        L.spec_verify_sample_timed.restype = I
        L.spec_verify_greedy_timed.argtypes = [P, LL, P, I, I, I, I, P, P, P, P, P, P, SZ, P, P, P]
        L.spec_verify_greedy_timed.restype = I
        L.spec_verify_candidates_timed.argtypes = [P, LL, P, P, I, I, I, I, I, I, I, P, P, P, P, P, SZ,
                                                   P, P, P]
        L.spec_verify_candidates_timed.restype = I
        _lib = L
    return _lib


EXPORTED = (
    "spec_verify_version", "spec_verify_status_string", "spec_verify_workspace_bytes",
    "spec_verify_greedy", "spec_verify_sample", "spec_verify_greedy_candidates",
    "spec_verify_greedy_ext", "spec_verify_sample_lenient", "spec_verify_greedy_candidates_ext",
    "spec_verify_greedy_tree", "spec_verify_sample_lazy", "spec_verify_greedy_lazy",
    "spec_verify_sample_truncated", "spec_verify_sample_timed", "spec_verify_greedy_timed",
    "spec_verify_candidates_timed", "spec_verify_sample_noalloc",
)


def hip_runtimes_loaded() -> list:
    """Paths of every libamdhip64 mapped into this process (must be exactly one)."""
    seen = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                seen.add(line.split()[-1])
    return sorted(seen)


def check_single_hip_runtime():
    rts = hip_runtimes_loaded()
    if len(rts) > 1:
        raise RuntimeError(f"more than one HIP runtime is loaded: {rts}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


# the current stream's raw handle without building a Stream object (about
# 0.1 us instead of 3 us per call)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device: torch.device):
    if stream is not None:
        if stream.device != device:
            raise ValueError(f"stream is on {stream.device}, the logits on {device}")
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _sv_dtype(dtype: torch.dtype) -> int:
    try:
        return _DTYPE[dtype]
    except KeyError:
        raise TypeError(f"logits must be float32, float16 or bfloat16, not {dtype}") from None


def workspace_bytes(B: int, rows_per_seq: int, V: int, dtype: torch.dtype) -> int:
    return int(lib().spec_verify_workspace_bytes(B, rows_per_seq, V, _sv_dtype(dtype)))


# The C ABI takes plain device pointers and cannot see buffer sizes, so every
# tensor is checked here before its pointer is passed: device, dtype, shape
# and layout.  A mismatch raises ValueError / TypeError and launches nothing.

def _describe(t) -> str:
    if not isinstance(t, torch.Tensor):
        return type(t).__name__
    return f"{t.dtype} {tuple(t.shape)} on {t.device}{'' if t.is_contiguous() else ', not contiguous'}"


def _need(t, name: str, shape: tuple, dtype: torch.dtype, device: torch.device):
    """A contiguous tensor of exactly this shape and dtype on the logits' device."""
    if (not isinstance(t, torch.Tensor) or t.device != device or t.dtype is not dtype
            or t.shape != shape or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on "
                         f"{device}; got {_describe(t)}")
    return t


def _logits(t, name: str, ndim: int, lead: Optional[tuple] = None, dtype=None) -> int:
    """Logits on the GPU, `ndim` dims, rows contiguous along V and evenly
    spaced over the leading dims; returns the row stride in elements."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on the GPU; got {_describe(t)}")
    if t.dim() != ndim or (lead is not None and tuple(t.shape[:-1]) != lead):
        want = f"[{', '.join(map(str, lead))}, V]" if lead is not None else f"{ndim} dims"
        raise ValueError(f"{name} must have shape {want}; got {tuple(t.shape)}")
    if dtype is not None and t.dtype is not dtype:
        raise TypeError(f"{name} must have the target's dtype {dtype}; got {t.dtype}")
    _sv_dtype(t.dtype)
    shape, strides = t.shape, t.stride()
    if strides[-1] != 1:
        raise ValueError(f"{name}: rows must be contiguous along the vocabulary")
    rs = strides[-2]
    expect = rs
    for d in range(ndim - 2, -1, -1):
        if shape[d] > 1 and strides[d] != expect:
            raise ValueError(f"{name} must be a [.., V] tensor whose rows are evenly spaced")
        expect *= shape[d]
    return rs


def _new(shape, dtype, device, owned: list):
    """A tensor the binding allocates for this call (listed in `owned`)."""
    t = torch.empty(shape, dtype=dtype, device=device)
    owned.append(t)
    return t


def _out(t, name: str, shape: tuple, dtype: torch.dtype, device: torch.device, owned: list):
    """A caller's output tensor, checked, or a new one (listed in `owned`)."""
    if t is None:
        return _new(shape, dtype, device, owned)
    return _need(t, name, shape, dtype, device)


def _workspace(ws, B, rows_per_seq, V, dtype, device, owned: list):
    """(tensor, size in bytes): the caller's contiguous device buffer, or a new
    one (listed in `owned`)."""
    if ws is None:
        need = workspace_bytes(B, rows_per_seq, V, dtype)
        ws = _new(max(need, 1), torch.uint8, device, owned)
    elif not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}; got {_describe(ws)}")
    return ws, ws.numel() * ws.element_size()


def _launched(stream, owned: list):
    """After a launch on a caller's `stream`: the tensors the binding allocated
    came from the current stream's pool, and the kernels on `stream` may still
    use them after this call returns (the workspace is even released at once).
    Recording them on `stream` keeps the caching allocator from handing their
    memory to other work before that stream's work is done."""
    if stream is None or not owned:
        return
    if stream == torch.cuda.current_stream(stream.device):
        return
    for t in owned:
        t.record_stream(stream)


def _event_handles(events, stream, device):
    """The raw HIP handles of a caller's pair of torch.cuda.Event objects
    (enable_timing=True), which the library records around the streaming
    kernel.  torch creates an event's handle at its first record, so an event
    never recorded is recorded once on the call's stream first."""
    if events is None:
        return None
    if len(events) != 2 or not all(isinstance(e, torch.cuda.Event) for e in events):
        raise ValueError("events must be a pair of torch.cuda.Event objects")
    st = stream if stream is not None else torch.cuda.current_stream(device)
    out = []
    for e in events:
        if not e.cuda_event:
            e.record(st)
        out.append(e.cuda_event)
    return out


def greedy(target: torch.Tensor, draft_tokens: torch.Tensor, *, out_tokens=None,
           out_num_accepted=None, workspace=None, stream=None, events=None):
    """Greedy verification.  target [B, k+1, V] (fp32/fp16/bf16, rows contiguous
    along V), draft_tokens [B, k] int32.  Returns (tokens [B, k+1], num_accepted [B])."""
    ts = _logits(target, "target", 3)
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    owned = []
    _need(draft_tokens, "draft_tokens", (B, k), torch.int32, dev)
    out_tokens = _out(out_tokens, "out_tokens", (B, k + 1), torch.int32, dev, owned)
    out_num_accepted = _out(out_num_accepted, "out_num_accepted", (B,), torch.int32, dev, owned)
    if B == 0:
        return out_tokens, out_num_accepted
    ws, wsb = _workspace(workspace, B, k + 1, V, target.dtype, dev, owned)
    ev = _event_handles(events, stream, dev)
    if ev is None:
        st = lib().spec_verify_greedy(_ptr(target), ts, _ptr(draft_tokens), B, k, V,
                                      _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_num_accepted),
                                      _ptr(ws), wsb, _stream(stream, dev))
    else:
        st = lib().spec_verify_greedy_timed(_ptr(target), ts, _ptr(draft_tokens), B, k, V,
                                            _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_num_accepted),
                                            None, None, None, _ptr(ws), wsb, _stream(stream, dev), *ev)
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_greedy")
    return out_tokens, out_num_accepted


def _sample_inputs(target, draft, draft_tokens, uniforms):
    """Checks the sampling entry points' inputs; returns (B, k, V, target
    row stride, draft row stride)."""
    ts = _logits(target, "target", 3)
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    if isinstance(draft, torch.Tensor) and draft.device != dev:
        raise ValueError(f"draft must be on the target's device {dev}; got {_describe(draft)}")
    ds = _logits(draft, "draft", 3, (B, k), target.dtype)
    _need(draft_tokens, "draft_tokens", (B, k), torch.int32, dev)
    _need(uniforms, "uniforms", (B, k + 1), torch.float32, dev)
    return B, k, V, ts, ds


def sample(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
           uniforms: torch.Tensor, temperature: float, *, return_probs: bool = False,
           out_tokens=None, out_num_accepted=None, out_p_x=None, out_q_x=None,
           workspace=None, stream=None, events=None):
    """Sampling verification.  target [B, k+1, V], draft [B, k, V] (same dtype),
    draft_tokens [B, k] int32, uniforms [B, k+1] float32 in [0, 1).
    Returns (tokens [B, k+1], num_accepted [B]) and, with return_probs,
    also (p_x [B, k], q_x [B, k])."""
    B, k, V, ts, ds = _sample_inputs(target, draft, draft_tokens, uniforms)
    dev = target.device
    owned = []
    out_tokens = _out(out_tokens, "out_tokens", (B, k + 1), torch.int32, dev, owned)
    out_num_accepted = _out(out_num_accepted, "out_num_accepted", (B,), torch.int32, dev, owned)
    if return_probs:
        out_p_x = _out(out_p_x, "out_p_x", (B, k), torch.float32, dev, owned)
        out_q_x = _out(out_q_x, "out_q_x", (B, k), torch.float32, dev, owned)
    else:
        out_p_x = None if out_p_x is None else _need(out_p_x, "out_p_x", (B, k), torch.float32, dev)
        out_q_x = None if out_q_x is None else _need(out_q_x, "out_q_x", (B, k), torch.float32, dev)
    if B == 0:
        return (out_tokens, out_num_accepted, out_p_x, out_q_x) if return_probs else (out_tokens, out_num_accepted)
    ws, wsb = _workspace(workspace, B, 2 * k + 1, V, target.dtype, dev, owned)
    ev = _event_handles(events, stream, dev)
    if ev is None:
        st = lib().spec_verify_sample(_ptr(target), ts, _ptr(draft), ds,
                                      _ptr(draft_tokens), _ptr(uniforms), float(temperature), B, k, V,
                                      _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_num_accepted),
                                      _ptr(out_p_x), _ptr(out_q_x), _ptr(ws), wsb, _stream(stream, dev))
    else:
        st = lib().spec_verify_sample_timed(_ptr(target), ts, _ptr(draft), ds, _ptr(draft_tokens),
                                            _ptr(uniforms), float(temperature), 1.0, 0, 1.0, B, k, V,
                                            _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_num_accepted),
                                            _ptr(out_p_x), _ptr(out_q_x), _ptr(ws), wsb, _stream(stream, dev),
                                            *ev)
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_sample")
    if return_probs:
        return out_tokens, out_num_accepted, out_p_x, out_q_x
    return out_tokens, out_num_accepted


def sample_noalloc(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                   uniforms: torch.Tensor, temperature: float, *, out_tokens, out_num_accepted,
                   out_p_x=None, out_q_x=None, stream=None):
    """`sample` for callers that cannot allocate: the outputs are the caller's
    (required), and the library's static scratch of NOALLOC_SCRATCH_BYTES per
    device replaces the workspace.  Calls that overlap on one device race on
    that scratch.  Returns (tokens, num_accepted)."""
    B, k, V, ts, ds = _sample_inputs(target, draft, draft_tokens, uniforms)
    dev = target.device
    _need(out_tokens, "out_tokens", (B, k + 1), torch.int32, dev)
    _need(out_num_accepted, "out_num_accepted", (B,), torch.int32, dev)
    for t, name in ((out_p_x, "out_p_x"), (out_q_x, "out_q_x")):
        if t is not None:
            _need(t, name, (B, k), torch.float32, dev)
    if B == 0:
        return out_tokens, out_num_accepted
    st = lib().spec_verify_sample_noalloc(_ptr(target), ts, _ptr(draft), ds, _ptr(draft_tokens),
                                          _ptr(uniforms), float(temperature), B, k, V,
                                          _sv_dtype(target.dtype), _ptr(out_tokens),
                                          _ptr(out_num_accepted), _ptr(out_p_x), _ptr(out_q_x),
                                          _stream(stream, dev))
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_sample_noalloc")
    return out_tokens, out_num_accepted


def greedy_ext(target: torch.Tensor, draft_tokens: torch.Tensor, *, workspace=None, stream=None, events=None):
    """Greedy verification plus its phrase-harvesting by-products.  Returns
    (tokens [B, k+1], num_accepted [B], target_argmax [B, k+1],
    match_mask [B] (int64 bit pattern of the uint64 mask), num_match [B])."""
    ts = _logits(target, "target", 3)
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    owned = []
    _need(draft_tokens, "draft_tokens", (B, k), torch.int32, dev)
    out_tokens = _new((B, k + 1), torch.int32, dev, owned)
    out_na = _new((B,), torch.int32, dev, owned)
    out_v = _new((B, k + 1), torch.int32, dev, owned)
    out_mask = _new((B,), torch.int64, dev, owned)
    out_cnt = _new((B,), torch.int32, dev, owned)
    if B == 0:
        return out_tokens, out_na, out_v, out_mask, out_cnt
    ws, wsb = _workspace(workspace, B, k + 1, V, target.dtype, dev, owned)
    ev = _event_handles(events, stream, dev)
    if ev is None:
        st = lib().spec_verify_greedy_ext(_ptr(target), ts, _ptr(draft_tokens), B, k, V,
                                          _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_na), _ptr(out_v),
                                          _ptr(out_mask), _ptr(out_cnt), _ptr(ws), wsb, _stream(stream, dev))
    else:
        st = lib().spec_verify_greedy_timed(_ptr(target), ts, _ptr(draft_tokens), B, k, V,
                                            _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_na),
                                            _ptr(out_v), _ptr(out_mask), _ptr(out_cnt), _ptr(ws), wsb,
                                            _stream(stream, dev), *ev)
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_greedy_ext")
    return out_tokens, out_na, out_v, out_mask, out_cnt


def sample_lenient(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                   uniforms: torch.Tensor, temperature: float, lenience: float, *,
                   return_probs: bool = False, workspace=None, stream=None, events=None):
    """Sampling verification with lenience l >= 1 (l = 1: `sample`)."""
    B, k, V, ts, ds = _sample_inputs(target, draft, draft_tokens, uniforms)
    dev = target.device
    owned = []
    out_tokens = _new((B, k + 1), torch.int32, dev, owned)
    out_na = _new((B,), torch.int32, dev, owned)
    out_p_x = _new((B, k), torch.float32, dev, owned) if return_probs else None
    out_q_x = _new((B, k), torch.float32, dev, owned) if return_probs else None
    if B == 0:
        return (out_tokens, out_na, out_p_x, out_q_x) if return_probs else (out_tokens, out_na)
    ws, wsb = _workspace(workspace, B, 2 * k + 1, V, target.dtype, dev, owned)
    ev = _event_handles(events, stream, dev)
    if ev is None:
        st = lib().spec_verify_sample_lenient(_ptr(target), ts, _ptr(draft), ds, _ptr(draft_tokens),
                                              _ptr(uniforms), float(temperature), float(lenience), B, k, V,
                                              _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_na),
                                              _ptr(out_p_x), _ptr(out_q_x), _ptr(ws), wsb,
                                              _stream(stream, dev))
    else:
        st = lib().spec_verify_sample_timed(_ptr(target), ts, _ptr(draft), ds, _ptr(draft_tokens),
                                            _ptr(uniforms), float(temperature), float(lenience), 0, 1.0, B, k,
                                            V, _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_na),
                                            _ptr(out_p_x), _ptr(out_q_x), _ptr(ws), wsb, _stream(stream, dev),
                                            *ev)
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_sample_lenient")
    if return_probs:
        return out_tokens, out_na, out_p_x, out_q_x
    return out_tokens, out_na


def sample_truncated(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                     uniforms: torch.Tensor, temperature: float, top_k: int = 0, top_p: float = 1.0,
                     *, return_probs: bool = False, workspace=None, stream=None, events=None):
    """Sampling verification on top-k / top-p truncated target and draft rows
    (top_k = 0 and top_p >= 1 switch the steps off)."""
    B, k, V, ts, ds = _sample_inputs(target, draft, draft_tokens, uniforms)
    dev = target.device
    owned = []
    out_tokens = _new((B, k + 1), torch.int32, dev, owned)
    out_na = _new((B,), torch.int32, dev, owned)
    out_p_x = _new((B, k), torch.float32, dev, owned) if return_probs else None
    out_q_x = _new((B, k), torch.float32, dev, owned) if return_probs else None
    if B == 0:
        return (out_tokens, out_na, out_p_x, out_q_x) if return_probs else (out_tokens, out_na)
    ws, wsb = _workspace(workspace, B, 2 * k + 1, V, target.dtype, dev, owned)
    ev = _event_handles(events, stream, dev)
    if ev is None:
        st = lib().spec_verify_sample_truncated(_ptr(target), ts, _ptr(draft), ds, _ptr(draft_tokens),
                                                _ptr(uniforms), float(temperature), int(top_k),
                                                float(top_p), B, k, V, _sv_dtype(target.dtype),
                                                _ptr(out_tokens), _ptr(out_na), _ptr(out_p_x),
                                                _ptr(out_q_x), _ptr(ws), wsb, _stream(stream, dev))
    else:
        st = lib().spec_verify_sample_timed(_ptr(target), ts, _ptr(draft), ds, _ptr(draft_tokens),
                                            _ptr(uniforms), float(temperature), 1.0, int(top_k), float(top_p),
                                            B, k, V, _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_na),
                                            _ptr(out_p_x), _ptr(out_q_x), _ptr(ws), wsb, _stream(stream, dev),
                                            *ev)
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_sample_truncated")
    if return_probs:
        return out_tokens, out_na, out_p_x, out_q_x
    return out_tokens, out_na


def _candidate_inputs(target, cand_tokens):
    """Checks the candidate entry points' inputs; returns (B, C, R, V, L,
    target row stride)."""
    ts = _logits(target, "target", 4)
    B, C, R, V = target.shape
    if not isinstance(cand_tokens, torch.Tensor) or cand_tokens.dim() != 3:
        raise ValueError(f"cand_tokens must be a [B, C, L] int32 tensor; got {_describe(cand_tokens)}")
    L = cand_tokens.shape[2]
    _need(cand_tokens, "cand_tokens", (B, C, L), torch.int32, target.device)
    return B, C, R, V, L, ts


def greedy_candidates_ext(target: torch.Tensor, cand_tokens: torch.Tensor, *, workspace=None,
                          stream=None, events=None):
    """Multi-candidate greedy verification plus the argmax of every scored row.
    Returns (tokens [B, L+1], A [B], best [B], target_argmax [B, C, R])."""
    B, C, R, V, L, ts = _candidate_inputs(target, cand_tokens)
    dev = target.device
    owned = []
    out_tokens = _new((B, L + 1), torch.int32, dev, owned)
    out_na = _new((B,), torch.int32, dev, owned)
    out_best = _new((B,), torch.int32, dev, owned)
    out_v = _new((B, C, R), torch.int32, dev, owned)
    if B == 0:
        return out_tokens, out_na, out_best, out_v
    ws, wsb = _workspace(workspace, B, C * R, V, target.dtype, dev, owned)
    ev = _event_handles(events, stream, dev)
    if ev is None:
        st = lib().spec_verify_greedy_candidates_ext(_ptr(target), ts, _ptr(cand_tokens),
                                                     B, C, L, R, V, _sv_dtype(target.dtype), _ptr(out_tokens),
                                                     _ptr(out_na), _ptr(out_best), _ptr(out_v), _ptr(ws),
                                                     wsb, _stream(stream, dev))
    else:
        st = lib().spec_verify_candidates_timed(_ptr(target), ts, _ptr(cand_tokens), None, 0, B, C, L, R, V,
                                                _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_na),
                                                _ptr(out_best), _ptr(out_v), _ptr(ws), wsb, _stream(stream,
                                                dev), *ev)
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_greedy_candidates_ext")
    return out_tokens, out_na, out_best, out_v


def sample_lazy(target: torch.Tensor, draft: torch.Tensor, draft_tokens: torch.Tensor,
                uniforms: torch.Tensor, temperature: float, *, out_tokens=None, out_num_accepted=None,
                workspace=None, stream=None):
    """Early-exit sampling verification: `sample`'s results, reading only the rows
    the rule looks at.  Returns (tokens [B, k+1], num_accepted [B])."""
    B, k, V, ts, ds = _sample_inputs(target, draft, draft_tokens, uniforms)
    dev = target.device
    owned = []
    out_tokens = _out(out_tokens, "out_tokens", (B, k + 1), torch.int32, dev, owned)
    out_num_accepted = _out(out_num_accepted, "out_num_accepted", (B,), torch.int32, dev, owned)
    if B == 0:
        return out_tokens, out_num_accepted
    ws, wsb = _workspace(workspace, B, 2 * k + 1, V, target.dtype, dev, owned)
    st = lib().spec_verify_sample_lazy(_ptr(target), ts, _ptr(draft), ds, _ptr(draft_tokens),
                                       _ptr(uniforms), float(temperature), B, k, V,
                                       _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_num_accepted),
                                       _ptr(ws), wsb, _stream(stream, dev))
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_sample_lazy")
    return out_tokens, out_num_accepted


def greedy_lazy(target: torch.Tensor, draft_tokens: torch.Tensor, *, out_tokens=None,
                out_num_accepted=None, workspace=None, stream=None):
    """Early-exit greedy verification: `greedy`'s results, reading only the rows
    the rule looks at.  Returns (tokens [B, k+1], num_accepted [B])."""
    ts = _logits(target, "target", 3)
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    owned = []
    _need(draft_tokens, "draft_tokens", (B, k), torch.int32, dev)
    out_tokens = _out(out_tokens, "out_tokens", (B, k + 1), torch.int32, dev, owned)
    out_num_accepted = _out(out_num_accepted, "out_num_accepted", (B,), torch.int32, dev, owned)
    if B == 0:
        return out_tokens, out_num_accepted
    ws, wsb = _workspace(workspace, B, k + 1, V, target.dtype, dev, owned)
    st = lib().spec_verify_greedy_lazy(_ptr(target), ts, _ptr(draft_tokens), B, k, V,
                                       _sv_dtype(target.dtype), _ptr(out_tokens), _ptr(out_num_accepted),
                                       _ptr(ws), wsb, _stream(stream, dev))
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_greedy_lazy")
    return out_tokens, out_num_accepted


def greedy_tree(nodes: torch.Tensor, cand_tokens: torch.Tensor, cand_rows: torch.Tensor, *,
                workspace=None, stream=None, events=None):
    """Multi-candidate greedy verification over a token tree.  nodes [B, N, V],
    cand_tokens [B, C, L] int32, cand_rows [B, C, R] int32 (node row per
    candidate position).  Returns (tokens [B, L+1], A [B], best [B])."""
    ns = _logits(nodes, "nodes", 3)
    B, N, V = nodes.shape
    dev = nodes.device
    owned = []
    for t, name in ((cand_tokens, "cand_tokens"), (cand_rows, "cand_rows")):
        if not isinstance(t, torch.Tensor) or t.dim() != 3 or t.shape[0] != B:
            raise ValueError(f"{name} must be a [B, C, *] int32 tensor; got {_describe(t)}")
    _, C, L = cand_tokens.shape
    R = cand_rows.shape[2]
    _need(cand_tokens, "cand_tokens", (B, C, L), torch.int32, dev)
    _need(cand_rows, "cand_rows", (B, C, R), torch.int32, dev)
    out_tokens = _new((B, L + 1), torch.int32, dev, owned)
    out_na = _new((B,), torch.int32, dev, owned)
    out_best = _new((B,), torch.int32, dev, owned)
    if B == 0:
        return out_tokens, out_na, out_best
    ws, wsb = _workspace(workspace, B, N, V, nodes.dtype, dev, owned)
    ev = _event_handles(events, stream, dev)
    if ev is None:
        st = lib().spec_verify_greedy_tree(_ptr(nodes), ns, N, _ptr(cand_tokens),
                                           _ptr(cand_rows), B, C, L, R, V, _sv_dtype(nodes.dtype),
                                           _ptr(out_tokens), _ptr(out_na), _ptr(out_best), _ptr(ws),
                                           wsb, _stream(stream, dev))
    else:
        st = lib().spec_verify_candidates_timed(_ptr(nodes), ns, _ptr(cand_tokens), _ptr(cand_rows), N, B, C,
                                                L, R, V, _sv_dtype(nodes.dtype), _ptr(out_tokens),
                                                _ptr(out_na), _ptr(out_best), None, _ptr(ws), wsb,
                                                _stream(stream, dev), *ev)
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_greedy_tree")
    return out_tokens, out_na, out_best


def greedy_candidates(target: torch.Tensor, cand_tokens: torch.Tensor, *, out_tokens=None,
                      out_num_accepted=None, out_best=None, workspace=None, stream=None, events=None):
    """Multi-candidate greedy verification.  target [B, C, R, V] with R = L or L+1,
    cand_tokens [B, C, L] int32.  Returns (tokens [B, L+1], A [B], best [B])."""
    B, C, R, V, L, ts = _candidate_inputs(target, cand_tokens)
    dev = target.device
    owned = []
    out_tokens = _out(out_tokens, "out_tokens", (B, L + 1), torch.int32, dev, owned)
    out_num_accepted = _out(out_num_accepted, "out_num_accepted", (B,), torch.int32, dev, owned)
    out_best = _out(out_best, "out_best", (B,), torch.int32, dev, owned)
    if B == 0:
        return out_tokens, out_num_accepted, out_best
    ws, wsb = _workspace(workspace, B, C * R, V, target.dtype, dev, owned)
    ev = _event_handles(events, stream, dev)
    if ev is None:
        st = lib().spec_verify_greedy_candidates(_ptr(target), ts, _ptr(cand_tokens),
                                                 B, C, L, R, V, _sv_dtype(target.dtype), _ptr(out_tokens),
                                                 _ptr(out_num_accepted), _ptr(out_best), _ptr(ws),
                                                 wsb, _stream(stream, dev))
    else:
        st = lib().spec_verify_candidates_timed(_ptr(target), ts, _ptr(cand_tokens), None, 0, B, C, L, R, V,
                                                _sv_dtype(target.dtype), _ptr(out_tokens),
                                                _ptr(out_num_accepted), _ptr(out_best), None, _ptr(ws), wsb,
                                                _stream(stream, dev), *ev)
    _launched(stream, owned)
    if st != SV_OK:
        raise SpecVerifyError(st, "spec_verify_greedy_candidates")
    return out_tokens, out_num_accepted, out_best


lib()
check_single_hip_runtime()
