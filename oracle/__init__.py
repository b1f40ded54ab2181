"""CPU oracle for the speculative-decoding verification step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import this package.  The oracle itself is
plain single-threaded C in double precision (``oracle.c``); it shares no code
with the GPU library and never calls it.  The rule it implements, with its
sources on the pages, is described in ``oracle.h``.

All array arguments are numpy arrays; logits are float32 (fp16 and bf16 inputs
convert to float32 exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

MUT_NONE = 0
MUT_RESIDUAL_IS_P = 1
MUT_RESIDUAL_IS_Q = 2
MUT_BONUS_FROM_Q = 3
MUT_RATIO_INVERTED = 4
MUT_RESIDUAL_SIGN = 5

MAX_K = 63


def build() -> str:
    """Compile ``oracle.c`` with plain gcc (no fast-math, no FMA contraction)."""
    cmd = [
        "gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-o", LIB_PATH, os.path.join(_HERE, "oracle.c"), "-lm",
    ]
    subprocess.run(cmd, check=True)
    return LIB_PATH


class Trace(ctypes.Structure):
    _fields_ = [
        ("evaluated", ctypes.c_int),
        ("num_accepted", ctypes.c_int),
        ("sample_kind", ctypes.c_int),
        ("sampled_token", ctypes.c_int),
        ("ratio", ctypes.c_double * (MAX_K + 1)),
        ("accept_margin", ctypes.c_double * (MAX_K + 1)),
        ("p_x", ctypes.c_double * (MAX_K + 1)),
        ("q_x", ctypes.c_double * (MAX_K + 1)),
        ("sample_total", ctypes.c_double),
        ("sample_lo", ctypes.c_double),
        ("sample_hi", ctypes.c_double),
        ("sample_margin", ctypes.c_double),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"oracle library not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        LL = ctypes.c_longlong
        D = ctypes.c_double
        L.oracle_greedy.argtypes = [P, LL, P, I, I, I, P, P]
        L.oracle_sample.argtypes = [P, LL, P, LL, P, P, D, I, I, I, P, P, P, I]
        L.oracle_greedy_candidates.argtypes = [P, LL, P, I, I, I, I, I, P, P, P]
        L.oracle_token_probs_seq.argtypes = [P, LL, P, LL, P, D, I, I, P, P]
        L.oracle_draw_interval.argtypes = [P, P, D, I, I, P, P, P]
        L.oracle_sample_lenient.argtypes = [P, LL, P, LL, P, P, D, D, I, I, I, P, P, P]
        L.oracle_greedy_matches.argtypes = [P, LL, P, I, I, I, P, P, P]
        L.oracle_row_argmax.argtypes = [P, LL, LL, I, P]
        L.oracle_greedy_tree.argtypes = [P, LL, I, P, P, I, I, I, I, I, P, P, P]
        L.oracle_sample_truncated.argtypes = [P, LL, P, LL, P, P, D, I, D, I, I, I, P, P, P, P]
        L.oracle_truncated_row.argtypes = [P, I, D, I, D, P, P]
        for f in ("oracle_greedy", "oracle_sample", "oracle_greedy_candidates",
                  "oracle_token_probs_seq", "oracle_trace_size", "oracle_draw_interval",
                  "oracle_sample_lenient", "oracle_greedy_matches", "oracle_row_argmax",
                  "oracle_greedy_tree", "oracle_sample_truncated", "oracle_truncated_row"):
            getattr(L, f).restype = I
        if L.oracle_trace_size() != ctypes.sizeof(Trace):
            raise RuntimeError("oracle_trace layout mismatch")
        _lib = L
    return _lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def greedy(target, draft_tokens):
    """target [B, k+1, V] float32, draft_tokens [B, k] -> (tokens [B, k+1], num_accepted [B])."""
    z = _f32(target)
    x = _i32(draft_tokens)
    B, k1, V = z.shape
    k = k1 - 1
    assert x.shape == (B, k)
    out = np.full((B, k + 1), -1, np.int32)
    na = np.zeros(B, np.int32)
    rc = lib().oracle_greedy(_ptr(z), V, _ptr(x), B, k, V, _ptr(out), _ptr(na))
    if rc:
        raise RuntimeError(f"oracle_greedy failed: {rc}")
    return out, na


def sample(target, draft, draft_tokens, uniforms, temperature, mutation=MUT_NONE, traces=False):
    """target [B,k+1,V], draft [B,k,V] float32, tokens [B,k], uniforms [B,k+1] float32.

    Returns (tokens [B,k+1], num_accepted [B]) and, if ``traces``, a list of
    per-sequence ``Trace`` records."""
    z = _f32(target)
    y = _f32(draft)
    x = _i32(draft_tokens)
    u = _f32(uniforms)
    B, k1, V = z.shape
    k = k1 - 1
    assert y.shape == (B, k, V) and x.shape == (B, k) and u.shape == (B, k + 1)
    out = np.full((B, k + 1), -1, np.int32)
    na = np.zeros(B, np.int32)
    tr = (Trace * B)() if traces else None
    rc = lib().oracle_sample(_ptr(z), V, _ptr(y), V, _ptr(x), _ptr(u), float(temperature),
                             B, k, V, _ptr(out), _ptr(na),
                             ctypes.cast(tr, ctypes.c_void_p) if traces else None, int(mutation))
    if rc:
        raise RuntimeError(f"oracle_sample failed: {rc}")
    if traces:
        return out, na, list(tr)
    return out, na


def sample_lenient(target, draft, draft_tokens, uniforms, temperature, lenience, traces=False):
    """The sampling rule with lenience l >= 1 (l = 1 is `sample`)."""
    z = _f32(target)
    y = _f32(draft)
    x = _i32(draft_tokens)
    u = _f32(uniforms)
    B, k1, V = z.shape
    k = k1 - 1
    out = np.full((B, k + 1), -1, np.int32)
    na = np.zeros(B, np.int32)
    tr = (Trace * B)() if traces else None
    rc = lib().oracle_sample_lenient(_ptr(z), V, _ptr(y), V, _ptr(x), _ptr(u), float(temperature),
                                     float(lenience), B, k, V, _ptr(out), _ptr(na),
                                     ctypes.cast(tr, ctypes.c_void_p) if traces else None)
    if rc:
        raise RuntimeError(f"oracle_sample_lenient failed: {rc}")
    if traces:
        return out, na, list(tr)
    return out, na


def greedy_matches(target, draft_tokens):
    """target [B, k+1, V], tokens [B, k] -> (v [B, k+1], match mask [B] uint64, #Match [B])."""
    z = _f32(target)
    x = _i32(draft_tokens)
    B, k1, V = z.shape
    k = k1 - 1
    v = np.zeros((B, k + 1), np.int32)
    mask = np.zeros(B, np.uint64)
    cnt = np.zeros(B, np.int32)
    rc = lib().oracle_greedy_matches(_ptr(z), V, _ptr(x), B, k, V, _ptr(v), _ptr(mask), _ptr(cnt))
    if rc:
        raise RuntimeError(f"oracle_greedy_matches failed: {rc}")
    return v, mask, cnt


def row_argmax(rows):
    """rows [..., V] -> argmax of every row, shape [...]."""
    z = _f32(rows)
    V = z.shape[-1]
    n = z.size // V
    out = np.zeros(n, np.int32)
    rc = lib().oracle_row_argmax(_ptr(z), V, n, V, _ptr(out))
    if rc:
        raise RuntimeError(f"oracle_row_argmax failed: {rc}")
    return out.reshape(z.shape[:-1])


def token_probs(target_seq, draft_seq, draft_tokens_seq, temperature):
    """One sequence: target [k+1,V], draft [k,V], tokens [k] -> (p_x [k], q_x [k]) float64."""
    z = _f32(target_seq)
    y = _f32(draft_seq)
    x = _i32(draft_tokens_seq)
    k1, V = z.shape
    k = k1 - 1
    px = np.zeros(k, np.float64)
    qx = np.zeros(k, np.float64)
    rc = lib().oracle_token_probs_seq(_ptr(z), V, _ptr(y), V, _ptr(x), float(temperature), k, V,
                                      _ptr(px), _ptr(qx))
    if rc:
        raise RuntimeError(f"oracle_token_probs_seq failed: {rc}")
    return px, qx


def draw_interval(target_row, draft_row, temperature, token):
    """(lo, hi, weight): where `token` sits in the cumulative distribution a
    round draws from (residual against `draft_row`, or p if draft_row is None)."""
    z = _f32(target_row)
    y = None if draft_row is None else _f32(draft_row)
    lo = ctypes.c_double()
    hi = ctypes.c_double()
    w = ctypes.c_double()
    rc = lib().oracle_draw_interval(_ptr(z), None if y is None else _ptr(y), float(temperature),
                                    z.shape[-1], int(token), ctypes.byref(lo), ctypes.byref(hi),
                                    ctypes.byref(w))
    if rc:
        raise RuntimeError(f"oracle_draw_interval failed: {rc}")
    return lo.value, hi.value, w.value


def greedy_candidates(target, cand_tokens, R=None):
    """target [B, C, R, V] float32, cand [B, C, L] -> (tokens [B, L+1], A [B], best [B])."""
    z = _f32(target)
    c = _i32(cand_tokens)
    B, C, Rz, V = z.shape
    L = c.shape[2]
    R = Rz if R is None else R
    assert Rz == R and c.shape == (B, C, L)
    out = np.full((B, L + 1), -1, np.int32)
    na = np.zeros(B, np.int32)
    best = np.zeros(B, np.int32)
    rc = lib().oracle_greedy_candidates(_ptr(z), V, _ptr(c), B, C, L, R, V,
                                        _ptr(out), _ptr(na), _ptr(best))
    if rc:
        raise RuntimeError(f"oracle_greedy_candidates failed: {rc}")
    return out, na, best


def greedy_tree(nodes, cand_tokens, cand_rows):
    """nodes [B, N, V] float32, cand [B, C, L], cand_rows [B, C, R] -> (tokens [B, L+1], A, best)."""
    z = _f32(nodes)
    c = _i32(cand_tokens)
    r = _i32(cand_rows)
    B, N, V = z.shape
    _, C, L = c.shape
    R = r.shape[2]
    out = np.full((B, L + 1), -1, np.int32)
    na = np.zeros(B, np.int32)
    best = np.zeros(B, np.int32)
    rc = lib().oracle_greedy_tree(_ptr(z), V, N, _ptr(c), _ptr(r), B, C, L, R, V,
                                  _ptr(out), _ptr(na), _ptr(best))
    if rc:
        raise RuntimeError(f"oracle_greedy_tree failed: {rc}")
    return out, na, best


def sample_truncated(target, draft, draft_tokens, uniforms, temperature, top_k=0, top_p=1.0,
                     traces=False):
    """The rule on top-k / top-p truncated p and q.  Returns (tokens, num_accepted)
    and, with traces, also (traces, trunc_margin [B])."""
    z = _f32(target)
    y = _f32(draft)
    x = _i32(draft_tokens)
    u = _f32(uniforms)
    B, k1, V = z.shape
    k = k1 - 1
    out = np.full((B, k + 1), -1, np.int32)
    na = np.zeros(B, np.int32)
    tr = (Trace * B)() if traces else None
    margin = np.ones(B, np.float64)
    rc = lib().oracle_sample_truncated(_ptr(z), V, _ptr(y), V, _ptr(x), _ptr(u), float(temperature),
                                       int(top_k), float(top_p), B, k, V, _ptr(out), _ptr(na),
                                       ctypes.cast(tr, ctypes.c_void_p) if traces else None,
                                       _ptr(margin))
    if rc:
        raise RuntimeError(f"oracle_sample_truncated failed: {rc}")
    if traces:
        return out, na, list(tr), margin
    return out, na


def truncated_row(z, temperature, top_k=0, top_p=1.0):
    """p' of one row and its top-p boundary margin."""
    zz = _f32(z)
    V = zz.shape[-1]
    p = np.zeros(V, np.float64)
    m = ctypes.c_double()
    rc = lib().oracle_truncated_row(_ptr(zz), V, float(temperature), int(top_k), float(top_p),
                                    _ptr(p), ctypes.byref(m))
    if rc:
        raise RuntimeError(f"oracle_truncated_row failed: {rc}")
    return p, m.value
