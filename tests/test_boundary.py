"""The C-ABI boundary without a GPU: the library loads, exports every symbol the
header declares, sizes its workspace, and rejects bad arguments on the host
before anything is launched (outputs untouched).  No call here reaches a
kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


@pytest.fixture(scope="module")
def sv():
    so = os.path.join(ROOT, "draft_verification_verify_amd", "libspecverify.so")
    if not os.path.exists(so):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_sv_build", os.path.join(ROOT, "draft_verification_verify_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    import draft_verification_verify_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", text)))


def test_header_symbols_exported(sv):
    names = declared_functions()
    assert len(names) == 17, names
    assert sorted(sv.EXPORTED) == names
    for n in names:
        assert hasattr(sv.lib(), n), n


def test_single_hip_runtime(sv):
    rts = sv.hip_runtimes_loaded()
    assert len(rts) == 1, rts


def test_status_strings_and_version(sv):
    L = sv.lib()
    assert L.spec_verify_version() >= 200
    for s in range(6):
        assert L.spec_verify_status_string(s).startswith(b"SV_")
    assert L.spec_verify_status_string(99) == b"unknown status"


def test_workspace_bytes(sv):
    L = sv.lib()
    ws = L.spec_verify_workspace_bytes
    assert ws(0, 5, 32000, 0) == 0
    assert ws(1, 0, 32000, 0) == 0
    assert ws(1, 5, 0, 0) == 0
    assert ws(1, 5, 32000, 7) == 0
    assert ws(1, 5, 1 << 29, 0) == 0
    for B, rps, V in [(1, 9, 32000), (64, 11, 32000), (256, 17, 128256), (32, 64, 152064),
                      (512, 33, 128256), (512, 17, 128256), (3, 2, 1), (7, 127, 13)]:
        n = ws(B, rps, V, 2)
        assert n > 0 and n % 256 == 0
        # enough for at least one 8-byte partial per row and the per-sequence state
        assert n >= B * rps * 8 + B * 32


# ---- error paths (host-side validation only) ---------------------------------
SENT = 0x5A5A5A5A


def host_buf(n):
    a = np.full(n, SENT, np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def fake(n=64):
    """A valid-looking non-null pointer; validation rejects before any use."""
    a = np.zeros(n, np.float32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def call_greedy(L, **kw):
    a = dict(target=fake()[1], stride=100, tokens=fake()[1], B=2, k=3, V=100, dt=2,
             out=None, nacc=None, ws=fake()[1], wsb=1 << 30, stream=None)
    a.update(kw)
    return L.spec_verify_greedy(a["target"], a["stride"], a["tokens"], a["B"], a["k"], a["V"], a["dt"],
                                a["out"], a["nacc"], a["ws"], a["wsb"], a["stream"])


def test_greedy_rejects_bad_arguments(sv):
    L = sv.lib()
    keep = []
    out, po = host_buf(64)
    nacc, pn = host_buf(8)
    keep += [out, nacc]
    base = dict(out=po, nacc=pn)
    cases = [
        (dict(target=None), sv.SV_EINVAL), (dict(tokens=None), sv.SV_EINVAL),
        (dict(out=None), sv.SV_EINVAL), (dict(nacc=None), sv.SV_EINVAL),
        (dict(B=0), sv.SV_EINVAL), (dict(k=0), sv.SV_EINVAL), (dict(k=64), sv.SV_EINVAL),
        (dict(V=0), sv.SV_EINVAL), (dict(stride=99), sv.SV_EINVAL), (dict(dt=3), sv.SV_EDTYPE),
        (dict(dt=-1), sv.SV_EDTYPE), (dict(ws=None), sv.SV_EWORKSPACE), (dict(wsb=16), sv.SV_EWORKSPACE),
    ]
    for kw, want in cases:
        args = dict(base)
        args.update(kw)
        assert call_greedy(L, **args) == want, kw
    assert (out == SENT).all() and (nacc == SENT).all()


def test_sample_rejects_bad_arguments(sv):
    L = sv.lib()
    out, po = host_buf(64)
    nacc, pn = host_buf(8)
    px, ppx = host_buf(64)
    f = fake()[1]

    def call(**kw):
        a = dict(target=f, ts=100, draft=f, ds=100, tokens=f, u=f, T=1.0, B=2, k=3, V=100, dt=1,
                 out=po, nacc=pn, px=ppx, qx=None, ws=f, wsb=1 << 30)
        a.update(kw)
        return L.spec_verify_sample(a["target"], a["ts"], a["draft"], a["ds"], a["tokens"], a["u"],
                                    a["T"], a["B"], a["k"], a["V"], a["dt"], a["out"], a["nacc"],
                                    a["px"], a["qx"], a["ws"], a["wsb"], None)

    cases = [
        (dict(draft=None), sv.SV_EINVAL), (dict(u=None), sv.SV_EINVAL), (dict(ds=50), sv.SV_EINVAL),
        (dict(T=0.0), sv.SV_EINVAL), (dict(T=-1.0), sv.SV_EINVAL), (dict(T=float("inf")), sv.SV_EINVAL),
        (dict(T=float("nan")), sv.SV_EINVAL), (dict(T=1e-45), sv.SV_EINVAL), (dict(k=64), sv.SV_EINVAL),
        (dict(B=-3), sv.SV_EINVAL), (dict(dt=9), sv.SV_EDTYPE), (dict(wsb=0), sv.SV_EWORKSPACE),
    ]
    for kw, want in cases:
        assert call(**kw) == want, kw
    assert (out == SENT).all() and (nacc == SENT).all() and (px == SENT).all()


def test_candidates_rejects_bad_arguments(sv):
    L = sv.lib()
    out, po = host_buf(64)
    f = fake()[1]

    def call(**kw):
        a = dict(target=f, stride=100, cand=f, B=2, C=8, L=8, R=8, V=100, dt=2, out=po, A=f, best=f,
                 ws=f, wsb=1 << 30)
        a.update(kw)
        return L.spec_verify_greedy_candidates(a["target"], a["stride"], a["cand"], a["B"], a["C"],
                                               a["L"], a["R"], a["V"], a["dt"], a["out"], a["A"],
                                               a["best"], a["ws"], a["wsb"], None)

    cases = [
        (dict(C=9), sv.SV_EINVAL), (dict(L=0), sv.SV_EINVAL), (dict(R=7), sv.SV_EINVAL),
        (dict(R=10), sv.SV_EINVAL), (dict(C=1, L=64, R=64), sv.SV_EINVAL), (dict(best=None), sv.SV_EINVAL),
        (dict(cand=None), sv.SV_EINVAL), (dict(stride=10), sv.SV_EINVAL), (dict(dt=5), sv.SV_EDTYPE),
        (dict(ws=None), sv.SV_EWORKSPACE),
        (dict(C=1 << 30, L=4, R=4), sv.SV_EINVAL),      # C * L overflows an int
    ]
    for kw, want in cases:
        assert call(**kw) == want, kw
    assert (out == SENT).all()
    # tree layout: missing row map, N < 1, bad R
    assert L.spec_verify_greedy_tree(f, 100, 5, f, None, 2, 2, 3, 3, 100, 2, po, f, f, f, 1 << 30,
                                     None) == sv.SV_EINVAL
    assert L.spec_verify_greedy_tree(f, 100, 0, f, f, 2, 2, 3, 3, 100, 2, po, f, f, f, 1 << 30,
                                     None) == sv.SV_EINVAL
    assert L.spec_verify_greedy_tree(f, 100, 5, f, f, 2, 2, 3, 5, 100, 2, po, f, f, f, 1 << 30,
                                     None) == sv.SV_EINVAL
    assert (out == SENT).all()


def test_noalloc_refuses_shapes_beyond_its_scratch(sv):
    """spec_verify_sample_noalloc refuses, before any HIP call, a shape whose
    workspace exceeds its static scratch, and names the limit; the header's
    limit is the binding's."""
    L = sv.lib()
    text = open(HEADER).read()
    m = re.search(r"#define SV_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == sv.NOALLOC_SCRATCH_BYTES
    f = ctypes.c_void_p(64)
    out = np.full(8, SENT, np.int32)
    po = out.ctypes.data_as(ctypes.c_void_p)
    need = L.spec_verify_workspace_bytes(4096, 33, 128256, 2)
    assert need > sv.NOALLOC_SCRATCH_BYTES
    assert L.spec_verify_sample_noalloc(f, 128256, f, 128256, f, f, 1.0, 4096, 16, 128256, 2, po, po,
                                        None, None, None) == sv.SV_ESCRATCH
    assert b"SV_NOALLOC_SCRATCH_BYTES" in L.spec_verify_status_string(sv.SV_ESCRATCH)
    assert L.spec_verify_workspace_bytes(512, 33, 128256, 2) <= sv.NOALLOC_SCRATCH_BYTES
    assert (out == SENT).all()


def test_timed_variants_need_both_events(sv):
    """The measurement variants take the caller's two events; a missing one is
    SV_EINVAL before anything else happens (no HIP call, outputs untouched)."""
    L = sv.lib()
    f = ctypes.c_void_p(64)
    out = np.full(8, SENT, np.int32)
    po = out.ctypes.data_as(ctypes.c_void_p)
    for e0, e1 in ((None, f), (f, None), (None, None)):
        assert L.spec_verify_sample_timed(f, 100, f, 100, f, f, 1.0, 1.0, 0, 1.0, 2, 3, 100, 2, po, po,
                                          None, None, f, 1 << 30, None, e0, e1) == sv.SV_EINVAL
        assert L.spec_verify_greedy_timed(f, 100, f, 2, 3, 100, 2, po, po, None, None, None, f, 1 << 30,
                                          None, e0, e1) == sv.SV_EINVAL
        assert L.spec_verify_candidates_timed(f, 100, f, None, 0, 2, 2, 3, 3, 100, 2, po, po, po, None, f,
                                              1 << 30, None, e0, e1) == sv.SV_EINVAL
    assert (out == SENT).all()


def test_binding_fails_loudly_without_library(tmp_path):
    """The package has no fallback: with the library absent, import raises."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "draft_verification_verify_amd"
    shutil.copytree(os.path.join(ROOT, "draft_verification_verify_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "csrc", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import draft_verification_verify_amd"],
                       cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr


def test_lenient_and_ext_reject_bad_arguments(sv):
    L = sv.lib()
    out, po = host_buf(64)
    f = fake()[1]

    def lenient(lv, **kw):
        a = dict(target=f, ts=100, draft=f, ds=100, tokens=f, u=f, T=1.0, B=2, k=3, V=100, dt=2,
                 out=po, nacc=f, ws=f, wsb=1 << 30)
        a.update(kw)
        return L.spec_verify_sample_lenient(a["target"], a["ts"], a["draft"], a["ds"], a["tokens"],
                                            a["u"], a["T"], lv, a["B"], a["k"], a["V"], a["dt"],
                                            a["out"], a["nacc"], None, None, a["ws"], a["wsb"], None)

    for lv in (0.999, 0.0, -2.0, float("inf"), float("nan")):
        assert lenient(lv) == sv.SV_EINVAL, lv
    assert lenient(2.0, wsb=8) == sv.SV_EWORKSPACE
    assert L.spec_verify_greedy_ext(f, 100, None, 2, 3, 100, 2, po, f, f, f, f, f, 1 << 30, None) == sv.SV_EINVAL
    assert L.spec_verify_greedy_ext(f, 100, f, 2, 0, 100, 2, po, f, f, f, f, f, 1 << 30, None) == sv.SV_EINVAL
    assert L.spec_verify_greedy_candidates_ext(f, 100, f, 2, 8, 8, 10, 100, 2, po, f, f, f, f, 1 << 30,
                                               None) == sv.SV_EINVAL
    assert (out == SENT).all()


def test_lazy_reject_bad_arguments(sv):
    L = sv.lib()
    out, po = host_buf(64)
    f = fake()[1]
    assert L.spec_verify_sample_lazy(f, 100, None, 100, f, f, 1.0, 2, 3, 100, 2, po, f, f, 1 << 30,
                                     None) == sv.SV_EINVAL
    assert L.spec_verify_sample_lazy(f, 100, f, 100, f, f, 0.0, 2, 3, 100, 2, po, f, f, 1 << 30,
                                     None) == sv.SV_EINVAL
    assert L.spec_verify_sample_lazy(f, 100, f, 100, f, f, 1.0, 2, 3, 100, 7, po, f, f, 1 << 30,
                                     None) == sv.SV_EDTYPE
    assert L.spec_verify_sample_lazy(f, 100, f, 100, f, f, 1.0, 2, 3, 100, 2, po, f, f, 8,
                                     None) == sv.SV_EWORKSPACE
    assert L.spec_verify_greedy_lazy(f, 99, f, 2, 3, 100, 2, po, f, f, 1 << 30, None) == sv.SV_EINVAL
    assert L.spec_verify_greedy_lazy(f, 100, f, 2, 64, 100, 2, po, f, f, 1 << 30, None) == sv.SV_EINVAL
    assert (out == SENT).all()


def test_truncated_reject_bad_arguments(sv):
    L = sv.lib()
    out, po = host_buf(64)
    f = fake()[1]

    def call(top_k, top_p, **kw):
        a = dict(target=f, ts=100, draft=f, ds=100, tokens=f, u=f, T=1.0, B=2, k=3, V=100, dt=2,
                 out=po, nacc=f, ws=f, wsb=1 << 30)
        a.update(kw)
        return L.spec_verify_sample_truncated(a["target"], a["ts"], a["draft"], a["ds"], a["tokens"],
                                              a["u"], a["T"], top_k, top_p, a["B"], a["k"], a["V"],
                                              a["dt"], a["out"], a["nacc"], None, None, a["ws"],
                                              a["wsb"], None)

    for tk, tp in ((-1, 1.0), (0, 0.0), (0, -0.5), (5, float("nan")), (-3, 0.9)):
        assert call(tk, tp) == sv.SV_EINVAL, (tk, tp)
    # the fixed-point kept mass bounds V when truncation is on, not when it is off
    assert call(50, 1.0, V=(1 << 23) + 1, ts=(1 << 23) + 1, ds=(1 << 23) + 1) == sv.SV_EINVAL
    assert call(0, 0.9, V=(1 << 23) + 1, ts=(1 << 23) + 1, ds=(1 << 23) + 1) == sv.SV_EINVAL
    assert call(50, 0.9, T=0.0) == sv.SV_EINVAL
    assert call(50, 0.9, dt=4) == sv.SV_EDTYPE
    assert call(50, 0.9, wsb=8) == sv.SV_EWORKSPACE
    assert call(0, 1.0, wsb=8) == sv.SV_EWORKSPACE
    assert (out == SENT).all()


def test_c_client_host_side():
    """A plain C99 program (no Python, no torch) links the library and checks
    the host side of the boundary through include/spec_verify.h alone."""
    import importlib.util
    import subprocess
    spec = importlib.util.spec_from_file_location(
        "_sv_build", os.path.join(ROOT, "draft_verification_verify_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    if not os.path.exists(b.CLIENT_BIN):
        b.build_client()
    r = subprocess.run([b.CLIENT_BIN], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "all checks passed" in r.stdout


def test_binding_checks_tensors_before_any_launch(sv):
    """The binding checks every tensor (device, dtype, shape, layout) before
    it passes a pointer to the C ABI, which cannot see buffer sizes."""
    import torch
    cpu = torch.device("cpu")
    t = torch.zeros((2, 3), dtype=torch.int32)
    assert sv._need(t, "x", (2, 3), torch.int32, cpu) is t
    for bad in (torch.zeros((2, 4), dtype=torch.int32),            # shape
                torch.zeros((2, 3), dtype=torch.int64),            # dtype
                torch.zeros((3, 2), dtype=torch.int32).t(),        # layout
                [[0, 0, 0], [0, 0, 0]]):                           # not a tensor
        with pytest.raises(ValueError):
            sv._need(bad, "x", (2, 3), torch.int32, cpu)
    with pytest.raises(TypeError):
        sv._sv_dtype(torch.float64)
    # logits must live on the GPU: CPU tensors are refused before the library is called
    z = torch.zeros((2, 5, 16))
    with pytest.raises(ValueError, match="GPU"):
        sv.sample(z, z[:, :4], torch.zeros((2, 4), dtype=torch.int32), torch.zeros((2, 5)), 1.0)
    with pytest.raises(ValueError, match="GPU"):
        sv.greedy(z, torch.zeros((2, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        sv.greedy_candidates(torch.zeros((2, 2, 3, 16)), torch.zeros((2, 2, 3), dtype=torch.int32))
